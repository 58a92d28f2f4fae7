// Log-mel frontend for gfx950: framing, Hann window, 512-point real FFT,
// power spectrum, mel projection and log, in one kernel.
//
// Method: "Nemotron 3.5 Transcribe: From Recorded Speech to Dataset Audits",
// section "How audio and speakers reach the language model" -- 16 kHz mono
// waveform, 128 log-mel features, 25 ms Hann window, 512-point FFT, 10 ms hop.
// Readings of the open points: frame t = samples [160 t, 160 t + 400), periodic
// Hann window, power |X_k|^2 for k = 0..256, Slaney mel bank (peak 1), natural
// log of (energy + 2^-24).
//
// One wavefront transforms one frame at a time; the workgroups are persistent
// and read the window, twiddle and mel tables from LDS, copied once per
// workgroup (from global memory each frame's loads would form a chain of
// dependent cache round trips).  The 400 real samples, zero-padded to
// 512, are packed as 256 complex values z[n] = s[2n] + i s[2n+1]; a radix-4
// Stockham FFT of length 256 (four stages, one radix-4 butterfly per lane per
// stage, ping-pong through LDS) gives Z, and the split
//   X[k] = (Z[k] + conj Z[-k]) / 2 - i W512^k (Z[k] - conj Z[-k]) / 2
// recovers the 257 non-negative bins.
//
// Precision: the window, transform, power and mel sums run in float64 (tables
// built on the host in float64); the mel energies are rounded to float32 for
// the log, whose result is float32.  Below
// 1 kHz the mel bands are narrower than one bin, so a band's energy can be a
// single bin's power; when that power is small, a float32 transform's absolute
// error (about 1e-6 of the frame's spectral norm) turns into a log error of
// order 1e-3.  In float64 that error is ~1e-11.  The cost is ~14 kflop of
// fp64 per frame, small next to the frame's 2.3 KB of memory traffic.
// Memory traffic is the audio read (frames overlap by 240 samples; the overlap
// is served from cache) plus the feature write.

#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace enc {

namespace {

constexpr int WAVES = 8;
constexpr int FB_LDS = 2048;   // clips whose frame offsets are searched in LDS

typedef Cpx c32;

__device__ __forceinline__ c32 cmul(c32 a, c32 b) {
  return {a.re * b.re - a.im * b.im, a.re * b.im + a.im * b.re};
}

// Clip index of packed frame g: largest b with base[b] <= g (base ascending).
template <typename P>
__device__ __forceinline__ int find_clip(P base, int batch, int64_t g) {
  int lo = 0, hi = batch - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if ((int64_t)base[mid] <= g) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Orders a wavefront's LDS accesses across lanes: the LDS executes one
// wavefront's operations in issue order, so a compiler barrier suffices.
__device__ __forceinline__ void wave_lds_sync() { asm volatile("" ::: "memory"); }

// Persistent: a workgroup copies the tables (and, for up to FB_LDS clips, the
// frame offsets) into LDS once, then each wavefront takes frames
// g = wave_id, wave_id + waves, ... .
template <bool STACKED>
__global__ __launch_bounds__(64 * WAVES) void logmel_kernel(
    const float* __restrict__ audio, int64_t audio_stride,
    const int32_t* __restrict__ n_frames,     // [batch] F_b
    const int32_t* __restrict__ frame_base,   // [batch] first packed frame (STACKED)
    int batch, int64_t f_max, int64_t total_frames,
    const FrontendTables* __restrict__ tab,
    float* __restrict__ out_f32,              // [batch, f_max, 128]   (!STACKED)
    bf16_t* __restrict__ out_bf16)            // [sum 8 P_b, 128]       (STACKED)
{
  __shared__ double s_hann[WIN];
  __shared__ c32 s_tw256[256];
  __shared__ c32 s_tw512[NBIN];
  __shared__ int32_t s_mel_start[NMEL], s_mel_count[NMEL], s_mel_off[NMEL];
  __shared__ double s_mel_w[MEL_NNZ_MAX];
  __shared__ int32_t s_fb[FB_LDS];
  // per wavefront: the transform in place; the power spectrum (257 doubles)
  // then overwrites its first half
  __shared__ c32 buf[WAVES][256];

  const int tid = threadIdx.x;
  for (int i = tid; i < WIN; i += 64 * WAVES) s_hann[i] = tab->hann[i];
  for (int i = tid; i < 256; i += 64 * WAVES) s_tw256[i] = tab->tw256[i];
  for (int i = tid; i < NBIN; i += 64 * WAVES) s_tw512[i] = tab->tw512[i];
  for (int i = tid; i < NMEL; i += 64 * WAVES) {
    s_mel_start[i] = tab->mel_start[i];
    s_mel_count[i] = tab->mel_count[i];
    s_mel_off[i] = tab->mel_offset[i];
  }
  for (int i = tid; i < MEL_NNZ_MAX; i += 64 * WAVES) s_mel_w[i] = tab->mel_w[i];
  const bool fb_in_lds = STACKED && batch <= FB_LDS;
  if (fb_in_lds)
    for (int i = tid; i < batch; i += 64 * WAVES) s_fb[i] = frame_base[i];
  __syncthreads();

  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int64_t stride = (int64_t)gridDim.x * WAVES;
  c32* fb = buf[wave];
  double* pw = reinterpret_cast<double*>(fb);

  // Frame g: clip, frame in clip, validity; its 400 samples (lane j holds
  // samples 2n, 2n + 1 of n = j + 64 r) are fetched one frame ahead.
  auto locate = [&](int64_t g, int& b, int64_t& t) __attribute__((always_inline)) {
    if (STACKED) {
      b = fb_in_lds ? find_clip(s_fb, batch, g) : find_clip(frame_base, batch, g);
      t = g - (fb_in_lds ? s_fb[b] : frame_base[b]);
    } else {
      b = (int)(g / f_max);
      t = g - (int64_t)b * f_max;
    }
  };
  auto fetch = [&](int64_t g, float (&xs)[8], bool& valid) __attribute__((always_inline)) {
    int b;
    int64_t t;
    locate(g, b, t);
    valid = t < n_frames[b];
    const float* x = audio + (int64_t)b * audio_stride + t * HOP;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int n = lane + 64 * r;
      // the row stride (longest clip) may be odd: two 4-byte loads
      const bool in = valid && n < WIN / 2;
      xs[2 * r] = in ? x[2 * n] : 0.f;
      xs[2 * r + 1] = in ? x[2 * n + 1] : 0.f;
    }
  };

  int64_t g = (int64_t)blockIdx.x * WAVES + wave;
  float xs[8];
  bool valid = false;
  if (g < total_frames) fetch(g, xs, valid);
  for (; g < total_frames; g += stride) {
    c32 v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int n = lane + 64 * r;
      v[r] = n < WIN / 2 ? c32{(double)xs[2 * r] * s_hann[2 * n],
                                (double)xs[2 * r + 1] * s_hann[2 * n + 1]}
                         : c32{0.0, 0.0};
    }
    const bool cur_valid = valid;
    if (g + stride < total_frames) fetch(g + stride, xs, valid);   // next frame's samples

#pragma unroll
    for (int stage = 0; stage < 4; ++stage) {
      const int ns = 1 << (2 * stage);           // 1, 4, 16, 64
      if (stage > 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = fb[lane + 64 * r];
        wave_lds_sync();   // every lane's reads before any lane's writes
      }
      const int k = lane & (ns - 1);
      const int step = k * (64 >> (2 * stage));  // twiddle index unit: 2 pi / 256
#pragma unroll
      for (int r = 1; r < 4; ++r) v[r] = cmul(v[r], s_tw256[(r * step) & 255]);
      const c32 a0 = {v[0].re + v[2].re, v[0].im + v[2].im};
      const c32 a1 = {v[0].re - v[2].re, v[0].im - v[2].im};
      const c32 a2 = {v[1].re + v[3].re, v[1].im + v[3].im};
      const c32 a3 = {v[1].im - v[3].im, v[3].re - v[1].re};   // -i (v1 - v3)
      const int base = (lane >> (2 * stage)) * (ns * 4) + k;
      fb[base] = {a0.re + a2.re, a0.im + a2.im};
      fb[base + ns] = {a1.re + a3.re, a1.im + a3.im};
      fb[base + 2 * ns] = {a0.re - a2.re, a0.im - a2.im};
      fb[base + 3 * ns] = {a1.re - a3.re, a1.im - a3.im};
      wave_lds_sync();
    }

    // Split the packed transform into the 257 real-input bins and take power
    // (all of Z is read before the power spectrum overwrites it).
    c32 za[5], zb[5];
#pragma unroll
    for (int r = 0; r < 5; ++r) {
      const int k = lane + 64 * r;
      za[r] = fb[k & 255];
      zb[r] = fb[(256 - k) & 255];
    }
    wave_lds_sync();
#pragma unroll
    for (int r = 0; r < 5; ++r) {
      const int k = lane + 64 * r;
      if (k <= 256) {
        const c32 a = za[r];
        const c32 bconj = {zb[r].re, -zb[r].im};
        const c32 e = {0.5 * (a.re + bconj.re), 0.5 * (a.im + bconj.im)};
        const c32 d = {0.5 * (a.re - bconj.re), 0.5 * (a.im - bconj.im)};
        // o = -i d, then X = e + W512^k o
        const c32 o = {d.im, -d.re};
        const c32 wo = cmul(s_tw512[k], o);
        const double xr = e.re + wo.re, xi = e.im + wo.im;
        pw[k] = xr * xr + xi * xi;
      }
    }
    wave_lds_sync();

#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int m = lane + 64 * r;
      float val = 0.f;
      if (cur_valid) {
        const int k0 = s_mel_start[m];
        const int cnt = s_mel_count[m];
        const double* wm = s_mel_w + s_mel_off[m];
        // bands span at most 12 bins here: the first 16 terms are unrolled
        // (independent LDS reads), in the same order as the plain sum
        double acc = 0.0;
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (i < cnt) acc += wm[i] * pw[k0 + i];
        for (int i = 16; i < cnt; ++i) acc += wm[i] * pw[k0 + i];
        // natural log of (energy + 2^-24), taken in fp32 on the sum rounded to
        // fp32: log2 in hardware (v_log_f32, ~1 ulp) times ln 2; the result's
        // absolute error is ~1e-6, against a 1e-3 tolerance
        val = __builtin_amdgcn_logf((float)(acc + 5.9604644775390625e-08)) *
              0.69314718055994531f;
      }
      if (STACKED) out_bf16[g * NMEL + m] = f32_to_bf16(val);
      else out_f32[g * NMEL + m] = val;
    }
    wave_lds_sync();   // this frame's reads of pw before the next frame's writes
  }
}

int g_fe_grid = 0;

// Workgroups of the persistent grid: as many as the LDS lets reside (two per
// CU) on every CU.
int frontend_grid() {
  if (g_fe_grid == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      g_fe_grid = 2 * n;
    else
      g_fe_grid = 512;
  }
  return g_fe_grid;
}

}  // namespace

hipError_t launch_logmel_padded(const float* audio, int64_t audio_stride, const int32_t* n_frames,
                                int batch, int64_t f_max, const FrontendTables* tab, float* out,
                                hipStream_t stream) {
  const int64_t total = (int64_t)batch * f_max;
  if (total == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((total + WAVES - 1) / WAVES, frontend_grid());
  logmel_kernel<false><<<dim3((unsigned)blocks), dim3(64 * WAVES), 0, stream>>>(
      audio, audio_stride, n_frames, nullptr, batch, f_max, total, tab, out, nullptr);
  return hipGetLastError();
}

hipError_t launch_logmel_stacked(const float* audio, int64_t audio_stride, const int32_t* n_frames,
                                 const int32_t* frame_base, int batch, int64_t total_frames,
                                 const FrontendTables* tab, bf16_t* out, hipStream_t stream) {
  if (total_frames == 0) return hipSuccess;
  const int64_t blocks =
      std::min<int64_t>((total_frames + WAVES - 1) / WAVES, frontend_grid());
  logmel_kernel<true><<<dim3((unsigned)blocks), dim3(64 * WAVES), 0, stream>>>(
      audio, audio_stride, n_frames, frame_base, batch, 0, total_frames, tab, nullptr, out);
  return hipGetLastError();
}

}  // namespace enc
