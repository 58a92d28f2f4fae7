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
// One wavefront transforms one frame.  The 400 real samples, zero-padded to
// 512, are packed as 256 complex values z[n] = s[2n] + i s[2n+1]; a radix-4
// Stockham FFT of length 256 (four stages, one radix-4 butterfly per lane per
// stage, ping-pong through LDS) gives Z, and the split
//   X[k] = (Z[k] + conj Z[-k]) / 2 - i W512^k (Z[k] - conj Z[-k]) / 2
// recovers the 257 non-negative bins.
//
// Precision: the window, transform, power and mel sums run in float64 (tables
// built on the host in float64), only the log is rounded to float32.  Below
// 1 kHz the mel bands are narrower than one bin, so a band's energy can be a
// single bin's power; when that power is small, a float32 transform's absolute
// error (about 1e-6 of the frame's spectral norm) turns into a log error of
// order 1e-3.  In float64 that error is ~1e-11.  The cost is ~14 kflop of
// fp64 per frame, small next to the frame's 2.3 KB of memory traffic.
// Memory traffic is the audio read (frames overlap by 240 samples; the overlap
// is served from cache) plus the feature write.

#include "common.h"
#include "kernels.h"

namespace enc {

namespace {

constexpr int WAVES = 4;

typedef Cpx c32;

__device__ __forceinline__ c32 cmul(c32 a, c32 b) {
  return {a.re * b.re - a.im * b.im, a.re * b.im + a.im * b.re};
}

// Clip index of packed frame g: largest b with base[b] <= g (base ascending).
__device__ __forceinline__ int find_clip(const int32_t* __restrict__ base, int batch, int64_t g) {
  int lo = 0, hi = batch - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if ((int64_t)base[mid] <= g) lo = mid; else hi = mid - 1;
  }
  return lo;
}

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
  __shared__ c32 buf[WAVES][2][256];
  __shared__ double pw[WAVES][NBIN + 3];

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int64_t g = (int64_t)blockIdx.x * WAVES + wave;
  const bool in_range = g < total_frames;

  int b = 0;
  int64_t t = 0;
  if (in_range) {
    if (STACKED) {
      b = find_clip(frame_base, batch, g);
      t = g - frame_base[b];
    } else {
      b = (int)(g / f_max);
      t = g - (int64_t)b * f_max;
    }
  }
  const bool valid = in_range && t < n_frames[b];

  // Stage-0 inputs straight from HBM: lane j takes z[j + 64 r], r = 0..3.
  c32 v[4];
  {
    const float* x = audio + (int64_t)b * audio_stride + t * HOP;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int n = lane + 64 * r;
      if (valid && n < WIN / 2) {
        // the row stride (longest clip) may be odd: two 4-byte loads
        const double s0 = x[2 * n], s1 = x[2 * n + 1];
        v[r] = {s0 * tab->hann[2 * n], s1 * tab->hann[2 * n + 1]};
      } else {
        v[r] = {0.0, 0.0};
      }
    }
  }

  int src = 0;
#pragma unroll
  for (int stage = 0; stage < 4; ++stage) {
    const int ns = 1 << (2 * stage);           // 1, 4, 16, 64
    if (stage > 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = buf[wave][src][lane + 64 * r];
    }
    const int k = lane & (ns - 1);
    const int step = k * (64 >> (2 * stage));  // twiddle index unit: 2 pi / 256
#pragma unroll
    for (int r = 1; r < 4; ++r) v[r] = cmul(v[r], tab->tw256[(r * step) & 255]);
    const c32 a0 = {v[0].re + v[2].re, v[0].im + v[2].im};
    const c32 a1 = {v[0].re - v[2].re, v[0].im - v[2].im};
    const c32 a2 = {v[1].re + v[3].re, v[1].im + v[3].im};
    const c32 a3 = {v[1].im - v[3].im, v[3].re - v[1].re};   // -i (v1 - v3)
    const int base = (lane >> (2 * stage)) * (ns * 4) + k;
    const int dst = src ^ 1;
    buf[wave][dst][base] = {a0.re + a2.re, a0.im + a2.im};
    buf[wave][dst][base + ns] = {a1.re + a3.re, a1.im + a3.im};
    buf[wave][dst][base + 2 * ns] = {a0.re - a2.re, a0.im - a2.im};
    buf[wave][dst][base + 3 * ns] = {a1.re - a3.re, a1.im - a3.im};
    src = dst;
    __syncthreads();
  }

  // Split the packed transform into the 257 real-input bins and take power.
  const c32* Z = buf[wave][src];
#pragma unroll
  for (int r = 0; r < 5; ++r) {
    const int k = lane + 64 * r;
    if (k <= 256) {
      const c32 a = Z[k & 255];
      const c32 zc = Z[(256 - k) & 255];
      const c32 bconj = {zc.re, -zc.im};
      const c32 e = {0.5 * (a.re + bconj.re), 0.5 * (a.im + bconj.im)};
      const c32 d = {0.5 * (a.re - bconj.re), 0.5 * (a.im - bconj.im)};
      // o = -i d, then X = e + W512^k o
      const c32 o = {d.im, -d.re};
      const c32 wo = cmul(tab->tw512[k], o);
      const double xr = e.re + wo.re, xi = e.im + wo.im;
      pw[wave][k] = xr * xr + xi * xi;
    }
  }
  __syncthreads();

  if (!in_range) return;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int m = lane + 64 * r;
    float val = 0.f;
    if (valid) {
      const int k0 = tab->mel_start[m];
      const int cnt = tab->mel_count[m];
      const double* wm = tab->mel_w + tab->mel_offset[m];
      double acc = 0.0;
      for (int i = 0; i < cnt; ++i) acc += wm[i] * pw[wave][k0 + i];
      val = (float)log(acc + 5.9604644775390625e-08);   // 2^-24 guard
    }
    if (STACKED) out_bf16[g * NMEL + m] = f32_to_bf16(val);
    else out_f32[g * NMEL + m] = val;
  }
}

}  // namespace

hipError_t launch_logmel_padded(const float* audio, int64_t audio_stride, const int32_t* n_frames,
                                int batch, int64_t f_max, const FrontendTables* tab, float* out,
                                hipStream_t stream) {
  const int64_t total = (int64_t)batch * f_max;
  if (total == 0) return hipSuccess;
  const int64_t blocks = (total + WAVES - 1) / WAVES;
  logmel_kernel<false><<<dim3((unsigned)blocks), dim3(64 * WAVES), 0, stream>>>(
      audio, audio_stride, n_frames, nullptr, batch, f_max, total, tab, out, nullptr);
  return hipGetLastError();
}

hipError_t launch_logmel_stacked(const float* audio, int64_t audio_stride, const int32_t* n_frames,
                                 const int32_t* frame_base, int batch, int64_t total_frames,
                                 const FrontendTables* tab, bf16_t* out, hipStream_t stream) {
  if (total_frames == 0) return hipSuccess;
  const int64_t blocks = (total_frames + WAVES - 1) / WAVES;
  logmel_kernel<true><<<dim3((unsigned)blocks), dim3(64 * WAVES), 0, stream>>>(
      audio, audio_stride, n_frames, frame_base, batch, 0, total_frames, tab, nullptr, out);
  return hipGetLastError();
}

}  // namespace enc
