// Row-wise inclusive/exclusive scan along the last axis of a contiguous
// [rows, n] array (metaltile-std src/mlx/scan.rs: header comment for the
// definitions, "Multi-op scan variants" for prod/min/max and their identities,
// "Inclusive product scan" / "Exclusive product scan" for the product).
//
// Mapping: one workgroup of WPR wave64s owns one row and walks it in chunks of
// WPR*64*K vectors of a 16-byte-aligned window (so ragged rows, whose starts
// are not 16-byte aligned, still move in full vectors except at their two
// ends); for long rows that do not start on a 128-byte line of `out`, the
// window starts at the line before the row, so that every load and store
// instruction covers whole lines.  Wave w takes the w-th run of 64*K vectors of a chunk, and load j of
// its lane l is vector j*64 + l of that run, so every load instruction covers
// 1 KiB of contiguous memory.  Per chunk:
//   1. every wave issues its K loads (unconditionally; past the row they read
//      zeros), then per load: each lane scans its E elements serially in the
//      accumulation type (float32 for every float input, as the page's kernels
//      cast each load), the 64 lane totals are scanned across the wave with
//      DPP, and the running wave total is carried from load to load;
//   2. wave totals meet in LDS (one barrier per chunk; double-buffered so the
//      next chunk needs no second barrier), giving each wave the combine of
//      the row before it;
//   3. outputs are formed as prefix (+) lane-local prefix, the exclusive
//      variant reading the lane-local prefix one slot earlier (the "one-slot
//      store shift" of that page), narrowed with round-to-nearest-even and
//      stored with the same vector layout.
#include "device.hpp"
#include "launch.hpp"

namespace sca {

template <class F, Op O, bool EXCL, int E, int WPR, int K>
__global__ __launch_bounds__(64 * WPR) void scan_rows_kernel(uintptr_t in_base, uintptr_t out_base,
                                                            int64_t row0, int64_t n, int64_t ph,
                                                            int line_align) {
  using S = typename F::S;
  using W = typename F::W;
  using IO = VecIO<S, E>;
  constexpr int64_t VB = (int64_t)E * sizeof(S);       // bytes per vector
  constexpr int64_t kWaveVecs = (int64_t)kWave * K;     // vectors per wave per chunk
  constexpr int64_t kChunkVecs = kWaveVecs * WPR;       // vectors per chunk
  __shared__ W s_tot[2][WPR];

  const int lane = lane_id(), wave = wave_id();
  const int64_t row = row0 + blockIdx.x;
  // valid window elements of this row, and the vectors that cover them
  const int64_t lo = row * n + ph, hi = lo + n;
  int64_t v_first = lo / E;
  const int64_t v_last = (hi - 1) / E;
  if (line_align) {
    // start the window on a 128-byte line of `out`, so that every load and
    // store instruction covers whole lines (a window on a 16-byte boundary
    // alone spreads each 1 KiB instruction over nine lines); the vectors
    // before lo read as the identity and are not stored
    constexpr int64_t LV = 128 / VB;                    // vectors per line
    const int64_t lvph = (int64_t)((out_base % 128) / VB);
    const int64_t al = (v_first + lvph) / LV * LV - lvph;
    if (al >= 0) v_first = al;
  }
  const W id = identity<O, W>();
  W carry = id;  // combine of the row before the current chunk
  int parity = 0;
  for (int64_t vb = v_first; vb <= v_last; vb += kChunkVecs) {
    const int64_t wb = vb + wave * kWaveVecs;           // this wave's first vector
    const int64_t left = v_last + 1 - wb;
    const int64_t nv = left <= 0 ? 0 : (left < kWaveVecs ? left : kWaveVecs);
    const Buf buf(in_base + wb * VB, nv * VB);
    typename IO::Raw raw[K];
#pragma unroll
    for (int j = 0; j < K; ++j) raw[j] = IO::load(buf, (uint32_t)((j * kWave + lane) * VB));

    // 1. within the wave: x[j] becomes the lane-local inclusive prefix and
    //    pre[j] the combine of the wave's elements before the lane's vector
    W x[K][E];
    W pre[K];
    W wtot = id;
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const int64_t jv = wb + j * kWave;
      if (jv * E >= lo && (jv + kWave) * E <= hi) {     // wave-uniform: all vectors full
        IO::template unpack<F>(raw[j], x[j]);
      } else {
        IO::template unpack_masked<F>(raw[j], (jv + lane) * E, lo, hi, id, x[j]);
      }
#pragma unroll
      for (int k = 1; k < E; ++k) x[j][k] = combine<O>(x[j][k - 1], x[j][k]);
      const W incl = wave_scan_incl<O>(x[j][E - 1]);
      pre[j] = combine<O>(wtot, wave_shift_excl<O>(incl));
      wtot = combine<O>(wtot, readlane(incl, kWave - 1));
    }

    // 2. across the waves of the chunk
    W wp = carry;
    if constexpr (WPR > 1) {
      if (lane == 0) s_tot[parity][wave] = wtot;
      __syncthreads();
      W all = carry;
#pragma unroll
      for (int w = 0; w < WPR; ++w) {
        const W t = s_tot[parity][w];
        if (w < wave) wp = combine<O>(wp, t);
        all = combine<O>(all, t);
      }
      carry = all;
      parity ^= 1;
    } else {
      carry = combine<O>(carry, wtot);
    }

    // 3. outputs
    auto out_vec = [&](int j, W (&y)[E]) {
      const W q = combine<O>(wp, pre[j]);
      if constexpr (EXCL) {
        y[0] = q;
#pragma unroll
        for (int k = 1; k < E; ++k) y[k] = combine<O>(q, x[j][k - 1]);
      } else {
#pragma unroll
        for (int k = 0; k < E; ++k) y[k] = combine<O>(q, x[j][k]);
      }
    };
    if (wb * E >= lo && (wb + kWaveVecs) * E <= hi) {   // wave-uniform: all vectors full
      // one buffer per 4 KiB of the run (the lane's offset plus an immediate)
#pragma unroll
      for (int j = 0; j < K; ++j) {
        const Buf ob(out_base + (wb + (j & ~3) * kWave) * VB, 4 * kWave * VB);
        W y[E];
        out_vec(j, y);
        IO::template store_full<F>(ob, (uint32_t)(((j & 3) * kWave + lane) * VB), y);
      }
    } else {
#pragma unroll
      for (int j = 0; j < K; ++j) {
        W y[E];
        out_vec(j, y);
        const int64_t v = wb + j * kWave + lane;
        if (v <= v_last) IO::template store<F>(out_base, v, lo, hi, y);
      }
    }
  }
}

// A dispatch counts its work-items in 32 bits per grid dimension, so one
// launch takes fewer than 2^32 / 512 rows (512 threads being the largest
// workgroup here); more rows go out as several launches, each told its first
// row (rows are independent, so the launches need no ordering between them).
constexpr int64_t kRowsPerLaunch = 1ll << 22;

template <class F, Op O, bool EXCL, int E, int WPR, int K>
static void launch_rows_cfg(uintptr_t in_base, uintptr_t out_base, int64_t rows, int64_t n,
                            int64_t ph, int line_align, hipStream_t stream) {
  static_assert(64 * WPR * kRowsPerLaunch < (1ll << 32), "a launch's work-items fit 32 bits");
  for (int64_t row0 = 0; row0 < rows; row0 += kRowsPerLaunch) {
    const int64_t nr = rows - row0 < kRowsPerLaunch ? rows - row0 : kRowsPerLaunch;
    scan_rows_kernel<F, O, EXCL, E, WPR, K><<<dim3((unsigned)nr), dim3(64 * WPR), 0, stream>>>(
        in_base, out_base, row0, n, ph, line_align);
  }
}

// Launch shape by the number of vectors a row's window can span, measured on
// MI355X for bf16 rows of 8192 elements (1024 vectors) and 8191 (up to 1032
// once the window starts on the line before the row): four waves of four
// loads for 1024 (42.4 us; one or two waves with several chunks per row
// 46-48 us), six waves of three for up to 1152 (44.9 us before the windows
// started on lines, against 48.1 for four waves of five, 46.2 for five of
// four and 55-56 for nine or ten waves of two).  When every row is resident
// at once (the fp32 [1024, 4096] rows: 1024 workgroups), two waves of eight
// loads finish sooner: 6.1 us against 6.4-6.65 for four of four, and 7.2-7.4
// for eight of two.  Between 256 and 768 vectors the shape follows the row
// (bf16 rows over 2^26 elements, us): 271 vectors 2x3 45.3 against 4x4
// 70.1 and 4x2 51.0; 333: 4x2 44.0, 2x3 45.0, 4x4 56.9; 383: 4x2 43.5, 4x4
// 50.7; 446: 4x2 44.1, 4x4 47.1; 520: 4x3 44.3, 4x4 45.2; 633: 4x3 44.0,
// 4x4 44.0; 758: 4x3 45.3, 4x4 44.7.
//
// Windows start on a line of `out` for rows of more than 256 vectors that do
// not all start on one: measured on bf16 [8192, 8192] rows shifted by 16 /
// 32 / 64 / 512 bytes, 45.0 / 44.8 / 43.8 / 42.9 us against 42.8 aligned.
// Shorter rows keep their shape (a line's slack could push them into the
// next one) and are short enough that few of their instructions straddle.
template <class F, Op O, bool EXCL, int E>
static hipError_t launch_rows_e(uintptr_t in_base, uintptr_t out_base, int64_t rows, int64_t n,
                                int64_t ph, hipStream_t stream) {
  using S = typename F::S;
  constexpr int64_t LV = 128 / ((int64_t)E * (int64_t)sizeof(S));   // vectors per line
  // vectors one row can touch: exactly n/E when every row starts on a vector
  // boundary, else one more for a row that straddles
  int64_t vmax = (ph == 0 && n % E == 0) ? n / E : (n + 2 * E - 2) / E;
  // every row starts on a line of out when the window does and rows are whole lines
  const bool on_lines = ph == 0 && out_base % 128 == 0 && (n * (int64_t)sizeof(S)) % 128 == 0;
  const int line_align = (!on_lines && vmax > 4 * kWave) ? 1 : 0;
  if (line_align) vmax += LV - 1;
  if (vmax <= kWave) {
    launch_rows_cfg<F, O, EXCL, E, 1, 1>(in_base, out_base, rows, n, ph, line_align, stream);
  } else if (vmax <= 4 * kWave) {
    launch_rows_cfg<F, O, EXCL, E, 2, 2>(in_base, out_base, rows, n, ph, line_align, stream);
  } else if (vmax <= 5 * kWave) {
    launch_rows_cfg<F, O, EXCL, E, 2, 3>(in_base, out_base, rows, n, ph, line_align, stream);
  } else if (vmax <= 8 * kWave) {
    launch_rows_cfg<F, O, EXCL, E, 4, 2>(in_base, out_base, rows, n, ph, line_align, stream);
  } else if (vmax <= 12 * kWave) {
    launch_rows_cfg<F, O, EXCL, E, 4, 3>(in_base, out_base, rows, n, ph, line_align, stream);
  } else if (vmax <= 16 * kWave && rows <= 2048) {
    launch_rows_cfg<F, O, EXCL, E, 2, 8>(in_base, out_base, rows, n, ph, line_align, stream);
  } else if (vmax <= 16 * kWave) {
    launch_rows_cfg<F, O, EXCL, E, 4, 4>(in_base, out_base, rows, n, ph, line_align, stream);
  } else if (vmax <= 18 * kWave) {
    launch_rows_cfg<F, O, EXCL, E, 6, 3>(in_base, out_base, rows, n, ph, line_align, stream);
  } else if (vmax <= 20 * kWave) {
    launch_rows_cfg<F, O, EXCL, E, 4, 5>(in_base, out_base, rows, n, ph, line_align, stream);
  } else {
    launch_rows_cfg<F, O, EXCL, E, 8, 4>(in_base, out_base, rows, n, ph, line_align, stream);
  }
  return hipGetLastError();
}

template <class F, Op O, bool EXCL>
static hipError_t launch_rows_t(const void* in, void* out, int64_t rows, int64_t n,
                                hipStream_t stream) {
  using S = typename F::S;
  constexpr int EV = 16 / (int)sizeof(S);
  const uintptr_t ia = (uintptr_t)in, oa = (uintptr_t)out;
  if (ia % 16 == oa % 16) {
    // common phase: 16-byte vectors over the aligned window
    const int64_t ph = (int64_t)((ia % 16) / sizeof(S));
    return launch_rows_e<F, O, EXCL, EV>(ia - ph * sizeof(S), oa - ph * sizeof(S), rows, n, ph,
                                         stream);
  }
  return launch_rows_e<F, O, EXCL, 1>(ia, oa, rows, n, 0, stream);
}

template <class F>
static hipError_t launch_rows_f(const void* in, void* out, int64_t rows, int64_t n, int op,
                                bool excl, hipStream_t stream) {
  switch (op) {
    case 0: return excl ? launch_rows_t<F, Op::Add, true>(in, out, rows, n, stream)
                        : launch_rows_t<F, Op::Add, false>(in, out, rows, n, stream);
    case 1: return excl ? launch_rows_t<F, Op::Min, true>(in, out, rows, n, stream)
                        : launch_rows_t<F, Op::Min, false>(in, out, rows, n, stream);
    case 2: return excl ? launch_rows_t<F, Op::Max, true>(in, out, rows, n, stream)
                        : launch_rows_t<F, Op::Max, false>(in, out, rows, n, stream);
    default: return excl ? launch_rows_t<F, Op::Mul, true>(in, out, rows, n, stream)
                         : launch_rows_t<F, Op::Mul, false>(in, out, rows, n, stream);
  }
}

hipError_t launch_scan_rows(const void* in, void* out, int64_t rows, int64_t n, Fmt fmt, int op,
                            bool exclusive, hipStream_t stream) {
  switch (fmt) {
    case Fmt::F32: return launch_rows_f<FmtF32>(in, out, rows, n, op, exclusive, stream);
    case Fmt::F16: return launch_rows_f<FmtF16>(in, out, rows, n, op, exclusive, stream);
    case Fmt::BF16: return launch_rows_f<FmtBF16>(in, out, rows, n, op, exclusive, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sca
