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
// Four frames per wavefront, 16 lanes per frame.  The 400 real samples,
// zero-padded to 512, are packed as 256 complex values z[n] = s[2n] + i s[2n+1]
// and transformed as a 16 x 16 decomposition, n = 16 n1 + n2, k = k1 + 16 k2:
// lane n2 holds z[16 n1 + n2] for all n1 and takes a 16-point DFT over n1 in
// registers (itself two radix-4 passes); the outputs are multiplied by
// W256^(n2 k1) and transposed through LDS, so that lane k1 holds the column
// k1 and a second 16-point DFT over n2 gives Z[k1 + 16 k2] in register k2.
// The split
//   X[k] = (Z[k] + conj Z[-k]) / 2 - i W512^k (Z[k] - conj Z[-k]) / 2
// recovers the 257 non-negative bins; X[k] and X[256 - k] come from the same
// pair (Z[k], Z[256 - k]), so lane j takes the pairs of its registers 0..7,
// whose partners (lane 16 - j, registers 15..8) arrive through LDS.
//
// Precision: the window, transform, split and power run in float64; the
// powers are then rounded to float32 and the mel sums, the 2^-24 guard and the
// log run in float32.  Below 1 kHz the mel bands are narrower than one bin, so
// a band's energy can be a single bin's power; when that power is small, a
// float32 transform's absolute error (about 1e-6 of the frame's spectral norm)
// would turn into a log error of order 1e-3.  In float64 that error is ~1e-11.
// Once a power is formed, rounding it (and the mel weights) to float32 is a
// relative change of 2^-24 in a sum of non-negative terms, so the log moves by
// ~1e-7.  Memory traffic is the audio read (frames overlap by 240 samples;
// the overlap is served from cache) plus the feature write.

#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace enc {

namespace {

constexpr int WAVES = 8;          // wavefronts per workgroup (one workgroup per CU)
constexpr int ROWS = 4;           // frames per wavefront, 16 lanes each
constexpr int FB_LDS = 1024;      // clips whose frame offsets are searched in LDS
constexpr int SLOT_ROW = 272;     // 16-byte LDS slots per frame: 16 x 17 (padded)
constexpr int P_ROW = 336;        // floats per frame of the power spectrum (336 = 16 mod 64)
constexpr int TAPS = 13;          // 16 n1 + n2 < 200 needs n1 <= 12

typedef Cpx c64;

__device__ __forceinline__ c64 cadd(c64 a, c64 b) { return {a.re + b.re, a.im + b.im}; }
__device__ __forceinline__ c64 csub(c64 a, c64 b) { return {a.re - b.re, a.im - b.im}; }
__device__ __forceinline__ c64 cmul(c64 a, c64 b) {
  return {a.re * b.re - a.im * b.im, a.re * b.im + a.im * b.re};
}

// 4-point DFT in place (W4 = -i).  U3ZERO: the last input is zero.
template <bool U3ZERO>
__device__ __forceinline__ void dft4(c64& u0, c64& u1, c64& u2, c64& u3) {
  const c64 s02 = cadd(u0, u2), d02 = csub(u0, u2);
  const c64 s13 = U3ZERO ? u1 : cadd(u1, u3);
  const c64 d13 = U3ZERO ? u1 : csub(u1, u3);
  u0 = cadd(s02, s13);
  u2 = csub(s02, s13);
  u1 = {d02.re + d13.im, d02.im - d13.re};   // d02 - i d13
  u3 = {d02.re - d13.im, d02.im + d13.re};   // d02 + i d13
}

// x * W16^m for the exponents m = b c (b, c = 1..3) of the 16-point DFT.
template <int M>
__device__ __forceinline__ c64 mul_w16(c64 x) {
  constexpr double C1 = 0.92387953251128675613;   // cos(pi / 8)
  constexpr double S1 = 0.38268343236508977173;   // sin(pi / 8)
  constexpr double R2 = 0.70710678118654752440;   // sqrt(1 / 2)
  if constexpr (M == 4) return {x.im, -x.re};
  else if constexpr (M == 2) return {R2 * (x.re + x.im), R2 * (x.im - x.re)};
  else if constexpr (M == 6) return {R2 * (x.im - x.re), -R2 * (x.re + x.im)};
  else {
    constexpr double wr = M == 1 ? C1 : M == 3 ? S1 : -C1;   // M == 9
    constexpr double wi = M == 1 ? -S1 : M == 3 ? -C1 : S1;
    return cmul(x, c64{wr, wi});
  }
}

// x * W32^r for r = 0..7 (r is a compile-time constant after unrolling).
__device__ __forceinline__ c64 mul_w32(int r, c64 x) {
  constexpr double R2 = 0.70710678118654752440;   // sqrt(1 / 2) = cos(pi / 4)
  constexpr double C1 = 0.98078528040323044913;   // cos(pi / 16)
  constexpr double S1 = 0.19509032201612826785;   // sin(pi / 16)
  constexpr double C2 = 0.92387953251128675613;   // cos(pi / 8)
  constexpr double S2 = 0.38268343236508977173;   // sin(pi / 8)
  constexpr double C3 = 0.83146961230254523708;   // cos(3 pi / 16)
  constexpr double S3 = 0.55557023301960222474;   // sin(3 pi / 16)
  switch (r) {   // W32^r = cos(pi r / 16) - i sin(pi r / 16)
    case 0: return x;
    case 1: return cmul(x, c64{C1, -S1});
    case 2: return cmul(x, c64{C2, -S2});
    case 3: return cmul(x, c64{C3, -S3});
    case 4: return {R2 * (x.re + x.im), R2 * (x.im - x.re)};
    case 5: return cmul(x, c64{S3, -C3});
    case 6: return cmul(x, c64{S2, -C2});
    default: return cmul(x, c64{S1, -C1});
  }
}

// 16-point DFT in place, natural order in and out: v[k] <- sum_n v[n] W16^(nk).
// n = 4a + b, k = c + 4d: 4-point DFTs over a, twiddles W16^(bc), 4-point
// DFTs over b.  TAIL_ZERO: v[13], v[14], v[15] are zero on entry.
template <bool TAIL_ZERO>
__device__ __forceinline__ void dft16(c64 (&v)[16]) {
  dft4<false>(v[0], v[4], v[8], v[12]);
#pragma unroll
  for (int b = 1; b < 4; ++b) dft4<TAIL_ZERO>(v[b], v[4 + b], v[8 + b], v[12 + b]);
  // v[4c + b] now holds the c-th output of column b
  v[5] = mul_w16<1>(v[5]);
  v[6] = mul_w16<2>(v[6]);
  v[7] = mul_w16<3>(v[7]);
  v[9] = mul_w16<2>(v[9]);
  v[10] = mul_w16<4>(v[10]);
  v[11] = mul_w16<6>(v[11]);
  v[13] = mul_w16<3>(v[13]);
  v[14] = mul_w16<6>(v[14]);
  v[15] = mul_w16<9>(v[15]);
#pragma unroll
  for (int c = 0; c < 4; ++c) dft4<false>(v[4 * c], v[4 * c + 1], v[4 * c + 2], v[4 * c + 3]);
  // v[4c + d] holds output c + 4d: transpose the 4 x 4 index
  c64 t[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) t[i] = v[i];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int d = 0; d < 4; ++d) v[c + 4 * d] = t[4 * c + d];
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

// Persistent: a workgroup copies the window, the mel weights (and, for up to
// FB_LDS clips, the frame offsets) into LDS once; each wavefront then takes
// frame quads q = wave_id, wave_id + waves, ... (frames 4q .. 4q + 3).
template <bool STACKED>
__global__ __launch_bounds__(64 * WAVES) void logmel_kernel(
    const float* __restrict__ audio, int64_t audio_stride, int pair_loads,
    const int32_t* __restrict__ n_frames,     // [batch] F_b
    const int32_t* __restrict__ frame_base,   // [batch] first packed frame (STACKED)
    int batch, int64_t f_max, int64_t total_frames,
    const FrontendTables* __restrict__ tab,
    float* __restrict__ out_f32,              // [batch, f_max, 128]   (!STACKED)
    bf16_t* __restrict__ out_bf16)            // [sum 8 P_b, 128]       (STACKED)
{
  __shared__ __align__(16) double s_hann[WIN + 16];
  __shared__ float s_melw[MEL_TRIP_TOTAL * 16];
  __shared__ int32_t s_fb[FB_LDS];
  // per wavefront and frame row: the transpose (16 x 17 slots), then the
  // partner exchange (16 x 9 slots), then the float32 power spectrum
  __shared__ c64 s_buf[WAVES][ROWS * SLOT_ROW];

  const int tid = threadIdx.x;
  for (int i = tid; i < WIN + 16; i += 64 * WAVES) s_hann[i] = tab->hann[i];
  for (int i = tid; i < MEL_TRIP_TOTAL * 16; i += 64 * WAVES) s_melw[i] = (&tab->mel_w4[0][0])[i];
  const bool fb_in_lds = STACKED && batch <= FB_LDS;
  if (fb_in_lds)
    for (int i = tid; i < batch; i += 64 * WAVES) s_fb[i] = frame_base[i];
  __syncthreads();

  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int row = lane >> 4;
  const int j = lane & 15;
  c64* rb = s_buf[wave] + row * SLOT_ROW;         // this frame's LDS slots
  // power spectrum, 257 floats (+ a slot per lane past them); the rows start
  // 16 banks apart, so that the four rows' float accesses do not collide
  float* pb = reinterpret_cast<float*>(s_buf[wave]) + row * P_ROW;

  // per lane: the inter-pass twiddle W256^(j k1) = W256^(j c) W64^(j d) for
  // k1 = c + 4d is formed from wa[c] = W256^(j c) and wb[d] = W256^(4 j d);
  // the split twiddle W512^(j + 16 r) = W512^j W32^r from w512 = W512^j
  c64 wa[4], wb[4];
#pragma unroll
  for (int c = 1; c < 4; ++c) {
    wa[c] = tab->tw256[j * c];
    wb[c] = tab->tw256[(4 * j * c) & 255];
  }
  const c64 w512 = tab->tw512[j];
  // per lane: the first bin read for each of its bands
  int mel_lo[MEL_GROUPS];
#pragma unroll
  for (int i = 0; i < MEL_GROUPS; ++i) mel_lo[i] = tab->mel_rstart[j + 16 * i];
  // bin 128 (lane 0's register 8) is its own partner; the other lanes write
  // that value to a slot past the spectrum that no band reads
  const int p128 = j == 0 ? 128 : NBIN + j;

  // Frame of this lane's row in quad q: its validity and samples (lane j holds
  // samples 2n, 2n + 1 of n = 16 n1 + j), fetched one quad ahead.  Invalid
  // frames and the taps past the window read in-bounds samples that the zero
  // window (or the zero output) discards.
  auto fetch = [&](int64_t q, float (&xs)[2 * TAPS], bool& ok) __attribute__((always_inline)) {
    const int64_t g = q * ROWS + row;
    int b = 0;
    int64_t t = 0;
    if (g < total_frames) {
      if (STACKED) {
        b = fb_in_lds ? find_clip(s_fb, batch, g) : find_clip(frame_base, batch, g);
        t = g - (fb_in_lds ? s_fb[b] : frame_base[b]);
      } else {
        b = (int)(g / f_max);
        t = g - (int64_t)b * f_max;
      }
    }
    ok = g < total_frames && t < n_frames[b];
    const float* x = ok ? audio + (int64_t)b * audio_stride + t * HOP : audio;
    if (pair_loads) {
#pragma unroll
      for (int n1 = 0; n1 < TAPS; ++n1) {
        const int n = min(16 * n1 + j, WIN / 2 - 1);
        const float2 p = *reinterpret_cast<const float2*>(x + 2 * n);
        xs[2 * n1] = p.x;
        xs[2 * n1 + 1] = p.y;
      }
    } else {
#pragma unroll
      for (int n1 = 0; n1 < TAPS; ++n1) {
        const int n = min(16 * n1 + j, WIN / 2 - 1);
        xs[2 * n1] = x[2 * n];
        xs[2 * n1 + 1] = x[2 * n + 1];
      }
    }
  };

  const int64_t n_quads = (total_frames + ROWS - 1) / ROWS;
  const int64_t qstride = (int64_t)gridDim.x * WAVES;
  int64_t q = (int64_t)blockIdx.x * WAVES + wave;
  float xs[2 * TAPS];
  bool ok = false;
  if (q < n_quads) fetch(q, xs, ok);
  for (; q < n_quads; q += qstride) {
    // windowed samples; the lane's taps are zero past WIN
    c64 v[16];
#pragma unroll
    for (int n1 = 0; n1 < TAPS; ++n1) {
      const double2 h = *reinterpret_cast<const double2*>(s_hann + 2 * (16 * n1 + j));
      v[n1] = {(double)xs[2 * n1] * h.x, (double)xs[2 * n1 + 1] * h.y};
    }
#pragma unroll
    for (int n1 = TAPS; n1 < 16; ++n1) v[n1] = {0.0, 0.0};
    const bool cur_ok = ok;
    const int64_t g = q * ROWS + row;
    if (q + qstride < n_quads) fetch(q + qstride, xs, ok);   // next quad's samples

    // pass 1 over n1, twiddles, transpose (write slot k1 * 17 + j, read j * 17 + n2)
    dft16<true>(v);
#pragma unroll
    for (int k1 = 1; k1 < 16; ++k1) {
      const int c = k1 & 3, d = k1 >> 2;
      const c64 t = c == 0 ? wb[d] : d == 0 ? wa[c] : cmul(wa[c], wb[d]);
      v[k1] = cmul(v[k1], t);
    }
#pragma unroll
    for (int k1 = 0; k1 < 16; ++k1) rb[k1 * 17 + j] = v[k1];
    wave_lds_sync();
#pragma unroll
    for (int n2 = 0; n2 < 16; ++n2) v[n2] = rb[j * 17 + n2];
    wave_lds_sync();
    // pass 2 over n2: v[k2] = Z[j + 16 k2]
    dft16<false>(v);

    // partners: lane j writes registers 8..15 to slots 9j + 0..7 and register
    // 0 to slot 9j + 8; the partner of Z[j + 16 r] (r < 8) is Z[256 - j - 16 r],
    // register 15 - r of lane 16 - j, or for lane 0 its own register 16 - r
#pragma unroll
    for (int s = 0; s < 8; ++s) rb[9 * j + s] = v[8 + s];
    rb[9 * j + 8] = v[0];
    wave_lds_sync();
    const c64* pr = rb + 9 * ((16 - j) & 15) + (j == 0 ? 1 : 0);
    c64 w[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) w[r] = pr[7 - r];
    wave_lds_sync();

    // split and power, times 4 (the mel weights carry the 1/4)
    double pk[8], pm[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const c64 a = v[r], b = w[r];
      const c64 e = {a.re + b.re, a.im - b.im};   // Z[k] + conj Z[-k]
      const c64 d = {a.re - b.re, a.im + b.im};   // Z[k] - conj Z[-k]
      const c64 wo = cmul(w512, mul_w32(r, c64{d.im, -d.re}));
      const double xr = e.re + wo.re, xi = e.im + wo.im;   // 2 X[k]
      const double yr = e.re - wo.re, yi = e.im - wo.im;   // 2 conj X[256 - k]
      pk[r] = xr * xr + xi * xi;
      pm[r] = yr * yr + yi * yi;
    }
    const double p_mid = 4.0 * (v[8].re * v[8].re + v[8].im * v[8].im);
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      pb[j + 16 * r] = (float)pk[r];
      pb[256 - j - 16 * r] = (float)pm[r];
    }
    pb[p128] = (float)p_mid;
    wave_lds_sync();

    // mel bands j + 16 i (all reads issued first), log, store
    float wv[MEL_TRIP_TOTAL], pv[MEL_TRIP_TOTAL];
#pragma unroll
    for (int t = 0; t < MEL_TRIP_TOTAL; ++t) wv[t] = s_melw[t * 16 + j];
    {
      int row0 = 0;
#pragma unroll
      for (int i = 0; i < MEL_GROUPS; ++i) {
#pragma unroll
        for (int t = 0; t < MEL_GROUP_TRIP[i]; ++t) pv[row0 + t] = pb[mel_lo[i] + t];
        row0 += MEL_GROUP_TRIP[i];
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    int row0 = 0;
#pragma unroll
    for (int i = 0; i < MEL_GROUPS; ++i) {
      float acc = 0.f;
#pragma unroll
      for (int t = 0; t < MEL_GROUP_TRIP[i]; ++t) acc = fmaf(wv[row0 + t], pv[row0 + t], acc);
      row0 += MEL_GROUP_TRIP[i];
      // natural log of (energy + 2^-24): log2 in hardware (v_log_f32, ~1 ulp)
      // times ln 2
      const float val =
          cur_ok ? __builtin_amdgcn_logf(acc + 5.9604644775390625e-08f) * 0.69314718055994531f
                 : 0.f;
      if (g < total_frames) {
        if (STACKED) out_bf16[g * NMEL + j + 16 * i] = f32_to_bf16(val);
        else out_f32[g * NMEL + j + 16 * i] = val;
      }
    }
    wave_lds_sync();   // this quad's reads of the spectrum before the next quad's writes
  }
}

int g_fe_grid = 0;

// Workgroups of the persistent grid: as many as the LDS lets reside (one per
// CU) on every CU.
int frontend_grid() {
  if (g_fe_grid == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      g_fe_grid = n;
    else
      g_fe_grid = 256;
  }
  return g_fe_grid;
}

// Two-float loads need every frame's first sample 8-byte aligned.
int pair_aligned(const float* audio, int64_t audio_stride) {
  return (audio_stride % 2 == 0) && (reinterpret_cast<uintptr_t>(audio) % 8 == 0);
}

}  // namespace

hipError_t launch_logmel_padded(const float* audio, int64_t audio_stride, const int32_t* n_frames,
                                int batch, int64_t f_max, const FrontendTables* tab, float* out,
                                hipStream_t stream) {
  const int64_t total = (int64_t)batch * f_max;
  if (total == 0) return hipSuccess;
  const int64_t quads = (total + ROWS - 1) / ROWS;
  const int64_t blocks = std::min<int64_t>((quads + WAVES - 1) / WAVES, frontend_grid());
  logmel_kernel<false><<<dim3((unsigned)blocks), dim3(64 * WAVES), 0, stream>>>(
      audio, audio_stride, pair_aligned(audio, audio_stride), n_frames, nullptr, batch, f_max,
      total, tab, out, nullptr);
  return hipGetLastError();
}

hipError_t launch_logmel_stacked(const float* audio, int64_t audio_stride, const int32_t* n_frames,
                                 const int32_t* frame_base, int batch, int64_t total_frames,
                                 const FrontendTables* tab, bf16_t* out, hipStream_t stream) {
  if (total_frames == 0) return hipSuccess;
  const int64_t quads = (total_frames + ROWS - 1) / ROWS;
  const int64_t blocks = std::min<int64_t>((quads + WAVES - 1) / WAVES, frontend_grid());
  logmel_kernel<true><<<dim3((unsigned)blocks), dim3(64 * WAVES), 0, stream>>>(
      audio, audio_stride, pair_aligned(audio, audio_stride), n_frames, frame_base, batch, 0,
      total_frames, tab, nullptr, out);
  return hipGetLastError();
}

}  // namespace enc
