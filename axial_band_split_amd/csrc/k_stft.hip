// The steps on either side of the core ([P1] "The forward chain", "Verified inference hot path"):
// a centred STFT (periodic Hann window of n_fft, reflect padding) of each chunk of a track into
// the core's input layout, the complex product of the core's masks with that STFT, the inverse
// STFT (windowed overlap-add divided by the summed squared window) and the faded overlap-add of
// the chunks (chunk, stride 0.9 chunk, linear fades of chunk/10, none at the track's two ends, a
// reflect pad of chunk - stride around tracks longer than twice that).
//
//   * one workgroup transforms one frame: the n_fft samples (or the one-sided spectrum, Hermitian-
//     completed) go into LDS and through a radix-2 Stockham FFT there (log2 n_fft stages, natural
//     order out, twiddles and window computed once per workgroup);
//   * every index map of the chunking (track reflect pad, chunk tail reflected or zeroed, the STFT's
//     own centre reflection) is applied while loading, so no padded copy of the track exists;
//   * the chunks' estimates are combined by a gather over output samples (at most two chunks and
//     ceil(n_fft / hop) frames meet at a sample), in stream order between groups of chunks: no
//     atomics, deterministic.
#include <mutex>

#include "kcommon.h"
#include "kernels.h"

namespace mbr {

// Frame buffer of the allocation-free inverse STFT (mbr_istft_masked_noalloc): one copy per GPU,
// at its own address on each, held until the process ends.  Host code never uses this name as an
// address: it asks the runtime for the current device's copy (istft_noalloc_scratch).
static __device__ __align__(256) char scratch[kIstftNoallocBytes];

namespace {

__device__ __forceinline__ int64_t reflect_idx(int64_t i, int64_t n) {
  if (n <= 1) return 0;
  const int64_t period = 2 * (n - 1);
  int64_t m = i % period;
  if (m < 0) m += period;
  return m < n ? m : period - m;
}

// sample s of the track at chunk-local position j (the chunk extended by the STFT's reflection)
__device__ __forceinline__ float fetch(const StftGeom& G, int chunk_idx, int s, int64_t j) {
  const int64_t C = G.chunk;
  j = reflect_idx(j, C);                                 // the STFT's centre padding
  const int64_t off = (int64_t)chunk_idx * G.stride;
  const int64_t n = min(C, G.Lp - off);
  int64_t p;
  if (j < n) p = off + j;
  else if (n > C / 2) p = off + reflect_idx(j, n);       // a tail over half a chunk: reflected
  else return 0.f;                                       // else zero-padded
  const int64_t t = G.pad ? reflect_idx(p - G.pad, G.L) : p;
  return G.wave[(int64_t)s * G.L + t];
}

__device__ __forceinline__ float2 cmul(float2 a, float2 b) {
  return make_float2(a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x);
}

// twiddles e^{-2 pi i k / N}, k < N/2, and the periodic Hann window: single-precision sin / cos
// of pi x (about one ulp) at arguments that are exact in float (N a power of two)
__device__ void tables(float2* tw, float* win, int N) {
  for (int k = threadIdx.x; k < N / 2; k += blockDim.x) {
    float sn, cs;
    sincospif(-2.0f * k / N, &sn, &cs);
    tw[k] = make_float2(cs, sn);
  }
  for (int i = threadIdx.x; i < N; i += blockDim.x) win[i] = 0.5f - 0.5f * cospif(2.0f * i / N);
}

// radix-2 Stockham FFT of N points from a into b (result in the returned buffer); inverse: e^{+i}
__device__ float2* fft(float2* a, float2* b, const float2* tw, int N, bool inverse) {
  for (int Ns = 1; Ns < N; Ns <<= 1) {
    const int step = N / (2 * Ns);
    for (int j = threadIdx.x; j < N / 2; j += blockDim.x) {
      const float2 v0 = a[j];
      const int k = j & (Ns - 1);
      float2 w = tw[k * step];
      if (inverse) w.y = -w.y;
      const float2 v1 = cmul(a[j + N / 2], w);
      const int d = ((j - k) << 1) + k;
      b[d] = make_float2(v0.x + v1.x, v0.y + v1.y);
      b[d + Ns] = make_float2(v0.x - v1.x, v0.y - v1.y);
    }
    __syncthreads();
    float2* t = a;
    a = b;
    b = t;
  }
  return a;
}

// grid (frames, channels, chunks of the group); out: [chunk][F*S][T][2]
__global__ __launch_bounds__(256) void stft_kernel(StftGeom G, float* spec) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int N = G.n_fft, F = N / 2 + 1, S = G.S;
  float2* a = (float2*)lds;
  float2* b = a + N;
  float2* tw = b + N;
  float* win = (float*)(tw + N / 2);
  tables(tw, win, N);
  __syncthreads();
  const int t = blockIdx.x, s = blockIdx.y, g = blockIdx.z;
  const int chunk_idx = G.chunk0 + g;
  for (int i = threadIdx.x; i < N; i += blockDim.x)
    a[i] = make_float2(fetch(G, chunk_idx, s, (int64_t)t * G.hop + i - N / 2) * win[i], 0.f);
  __syncthreads();
  const float2* X = fft(a, b, tw, N, false);
  float* dst = spec + (int64_t)g * F * S * G.T * 2;
  for (int k = threadIdx.x; k < F; k += blockDim.x)
    *(float2*)(dst + (((int64_t)k * S + s) * G.T + t) * 2) = X[k];
}

// grid (frames, channels * stems, chunks of the group); frames out: [chunk][stem][s][T][N]
__global__ __launch_bounds__(256) void istft_frames_kernel(StftGeom G, const float* spec, const float* masks,
                                                           int stems, float* frames) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int N = G.n_fft, F = N / 2 + 1, S = G.S, T = G.T;
  float2* a = (float2*)lds;
  float2* b = a + N;
  float2* tw = b + N;
  float* win = (float*)(tw + N / 2);
  tables(tw, win, N);
  const int t = blockIdx.x, s = blockIdx.y % S, stem = blockIdx.y / S, g = blockIdx.z;
  const float* sp = spec + (int64_t)g * F * S * T * 2;
  const float* mk = masks + ((int64_t)g * stems + stem) * F * S * T * 2;
  for (int k = threadIdx.x; k < F; k += blockDim.x) {
    const int64_t o = (((int64_t)k * S + s) * T + t) * 2;
    float2 x = cmul(*(const float2*)(sp + o), *(const float2*)(mk + o));
    if (k == 0 || k == N / 2) x.y = 0.f;                 // a real transform ignores these parts
    a[k] = x;
    if (k > 0 && k < N / 2) a[N - k] = make_float2(x.x, -x.y);
  }
  __syncthreads();
  const float2* y = fft(a, b, tw, N, true);
  float* dst = frames + ((((int64_t)g * stems + stem) * S + s) * T + t) * N;
  const float inv = 1.0f / N;
  for (int i = threadIdx.x; i < N; i += blockDim.x) dst[i] = y[i].x * inv * win[i];
}

__device__ __forceinline__ float hann_at(int i, int N) { return 0.5f - 0.5f * cospif(2.0f * i / N); }

// fade window of chunk c at local position j (linear, endpoints included; none at the track ends)
__device__ __forceinline__ float fade_at(const StftGeom& G, int c, int64_t j) {
  if (G.no_fade) return 1.f;
  const int64_t fade = G.chunk / 10;
  const bool first = c == 0, last = (int64_t)c * G.stride + G.stride >= G.Lp;
  if (!first && j < fade) return (float)((double)j / (double)(fade - 1));
  if (!last && j >= G.chunk - fade) return (float)(1.0 - (double)(j - (G.chunk - fade)) / (double)(fade - 1));
  return 1.f;
}

// For padded-track samples of the group's chunks: each chunk's inverse STFT at that sample
// (overlap-add of its frames over the summed squared window), faded, added to out / counter.
// grid.x covers [lo, hi); grid.y = stem * S + s.
__global__ __launch_bounds__(256) void ola_kernel(StftGeom G, const float* frames, int stems, int ngroup,
                                                  int64_t lo, int64_t hi, float* out, float* counter) {
  const int64_t n = lo + (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (n >= hi) return;
  const int N = G.n_fft, T = G.T, S = G.S;
  const int stem = blockIdx.y / S, s = blockIdx.y % S;
  float acc = 0.f, cnt = 0.f;
  for (int g = 0; g < ngroup; ++g) {
    const int c = G.chunk0 + g;
    const int64_t off = (int64_t)c * G.stride;
    const int64_t nv = min(G.chunk, G.Lp - off);
    const int64_t j = n - off;
    if (j < 0 || j >= nv) continue;
    // frames t with 0 <= j + N/2 - t*hop < N
    const int64_t q = j + N / 2;
    const int t_hi = (int)min((int64_t)T - 1, q / G.hop);
    const int t_lo = (int)max((int64_t)0, (q - N + G.hop) / G.hop);
    const float* fr = frames + (((int64_t)g * stems + stem) * S + s) * T * N;
    float y = 0.f, env = 0.f;
    for (int t = t_lo; t <= t_hi; ++t) {
      const int i = (int)(q - (int64_t)t * G.hop);
      if (i < 0 || i >= N) continue;
      const float w = hann_at(i, N);
      y += fr[(int64_t)t * N + i];
      env += w * w;
    }
    const float f = fade_at(G, c, j);
    acc += (y / env) * f;
    cnt += f;
  }
  out[((int64_t)stem * S + s) * G.Lp + n] += acc;
  if (counter && blockIdx.y == 0) counter[n] += cnt;
}

__global__ __launch_bounds__(256) void finish_kernel(StftGeom G, int stems, const float* out, const float* counter,
                                                     float* dst) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= G.L) return;
  const int row = blockIdx.y;                                   // stem * S + s
  const int64_t p = i + G.pad;
  dst[(int64_t)row * G.L + i] = out[(int64_t)row * G.Lp + p] / fmaxf(counter[p], 1e-8f);
}

size_t fft_lds(int N) { return (size_t)N * 2 * 8 + (size_t)N / 2 * 8 + (size_t)N * 4; }

__global__ void fill_kernel(float* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

}  // namespace

bool stft_supported(int n_fft) { return n_fft >= 16 && n_fft <= 4096 && (n_fft & (n_fft - 1)) == 0; }

hipError_t launch_stft(const StftGeom& G, int ngroup, float* spec, hipStream_t stream) {
  if (!stft_supported(G.n_fft) || G.T < 1 || ngroup < 1) return hipErrorInvalidValue;
  const size_t lds = fft_lds(G.n_fft);
  hipError_t e = hipFuncSetAttribute((const void*)stft_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(stft_kernel, dim3(G.T, G.S, ngroup), dim3(256), lds, stream, G, spec);
  return hipGetLastError();
}

hipError_t launch_istft_frames(const StftGeom& G, int ngroup, const float* spec, const float* masks, int stems,
                               float* frames, hipStream_t stream) {
  if (!stft_supported(G.n_fft) || G.T < 1 || ngroup < 1 || stems < 1) return hipErrorInvalidValue;
  const size_t lds = fft_lds(G.n_fft);
  hipError_t e = hipFuncSetAttribute((const void*)istft_frames_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(istft_frames_kernel, dim3(G.T, G.S * stems, ngroup), dim3(256), lds, stream, G, spec, masks,
                     stems, frames);
  return hipGetLastError();
}

hipError_t launch_ola(const StftGeom& G, const float* frames, int stems, int ngroup, int64_t lo, int64_t hi,
                      float* out, float* counter, hipStream_t stream) {
  if (hi <= lo) return hipSuccess;
  hipLaunchKernelGGL(ola_kernel, dim3((unsigned)((hi - lo + 255) / 256), stems * G.S), dim3(256), 0, stream, G,
                     frames, stems, ngroup, lo, hi, out, counter);
  return hipGetLastError();
}

hipError_t launch_finish(const StftGeom& G, int stems, const float* out, const float* counter, float* dst,
                         hipStream_t stream) {
  hipLaunchKernelGGL(finish_kernel, dim3((unsigned)((G.L + 255) / 256), stems * G.S), dim3(256), 0, stream, G,
                     stems, out, counter, dst);
  return hipGetLastError();
}

hipError_t istft_noalloc_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {   // once per device, with that device current
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_fill0(float* p, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

}  // namespace mbr
