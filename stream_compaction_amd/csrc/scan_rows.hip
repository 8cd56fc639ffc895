// Row-wise inclusive/exclusive scan along the last axis of a contiguous
// [rows, n] array (metaltile-std src/mlx/scan.rs: header comment for the
// definitions, "Multi-op scan variants" for min/max and their identities).
//
// Mapping: one wave64 owns one row; a 256-thread workgroup holds four rows.
// A row is read as consecutive 16-byte vectors of a window aligned to 16
// bytes (so ragged rows, whose starts are not 16-byte aligned, still move in
// full vectors except at their two ends).  Per chunk of 64*K vectors the wave
// issues all K loads first (load j of lane l is vector j*64 + l, so every
// load instruction covers 1 KiB of contiguous memory), then per load:
//   1. each lane scans its E elements serially in the accumulation type
//      (float32 for every float input, as the page's kernels cast each load);
//   2. the 64 lane totals are scanned across the wave with DPP
//      (wave_scan_incl), then shifted one lane for the exclusive offsets;
//   3. the running row prefix (`carry`, wave-uniform) is combined in front;
//   4. outputs are formed as prefix (+) lane-local prefix, with the exclusive
//      variant reading the lane-local prefix one slot earlier (the "one-slot
//      store shift" of that page), narrowed with round-to-nearest-even and
//      stored with the same vector layout.
// No LDS and no barrier: the rows of a workgroup are independent.
#include "device.hpp"
#include "launch.hpp"

namespace sca {

template <class F, Op O, bool EXCL, int E, int K>
__global__ __launch_bounds__(256) void scan_rows_kernel(uintptr_t in_base, uintptr_t out_base,
                                                       int64_t rows, int64_t n, int64_t ph) {
  using S = typename F::S;
  using W = typename F::W;
  using IO = VecIO<S, E>;
  const int lane = lane_id();
  const int64_t row = (int64_t)blockIdx.x * 4 + wave_id();
  if (row >= rows) return;
  // valid window elements of this row, and the vectors that cover them
  const int64_t lo = row * n + ph, hi = lo + n;
  const int64_t v_first = lo / E, v_last = (hi - 1) / E;
  const W id = identity<O, W>();
  const S id_s = narrow<F>(id);
  W carry = id;
  for (int64_t vb = v_first; vb <= v_last; vb += (int64_t)kWave * K) {
    // all loads of the chunk first, kept as raw storage bits
    typename IO::Raw raw[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const int64_t v = vb + j * kWave + lane;
      if (v <= v_last) raw[j] = IO::load(in_base, v, lo, hi, id_s);
    }
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const int64_t v = vb + j * kWave + lane;
      W x[E];
      if (v <= v_last) {
        IO::template unpack<F>(raw[j], x);
      } else {
#pragma unroll
        for (int k = 0; k < E; ++k) x[k] = id;
      }
      // 1. lane-serial inclusive prefix, in place
#pragma unroll
      for (int k = 1; k < E; ++k) x[k] = combine<O>(x[k - 1], x[k]);
      // 2. across the wave
      const W incl = wave_scan_incl<O>(x[E - 1]);
      const W excl = wave_shift_excl<O>(incl);
      // 3. everything before this lane's vector
      const W pre = combine<O>(carry, excl);
      carry = combine<O>(carry, readlane(incl, kWave - 1));
      // 4. outputs
      W y[E];
      if constexpr (EXCL) {
        y[0] = pre;
#pragma unroll
        for (int k = 1; k < E; ++k) y[k] = combine<O>(pre, x[k - 1]);
      } else {
#pragma unroll
        for (int k = 0; k < E; ++k) y[k] = combine<O>(pre, x[k]);
      }
      if (v <= v_last) IO::template store<F>(out_base, v, lo, hi, y);
    }
  }
}

template <class F, Op O, bool EXCL, int E>
static hipError_t launch_rows_e(uintptr_t in_base, uintptr_t out_base, int64_t rows, int64_t n,
                                int64_t ph, hipStream_t stream) {
  const int64_t vmax = (n + 2 * E - 2) / E;  // vectors one row can touch
  const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
  if (vmax <= kWave) {
    scan_rows_kernel<F, O, EXCL, E, 1><<<grid, block, 0, stream>>>(in_base, out_base, rows, n, ph);
  } else if (vmax <= 4 * kWave) {
    scan_rows_kernel<F, O, EXCL, E, 4><<<grid, block, 0, stream>>>(in_base, out_base, rows, n, ph);
  } else {
    scan_rows_kernel<F, O, EXCL, E, 17><<<grid, block, 0, stream>>>(in_base, out_base, rows, n, ph);
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
    default: return excl ? launch_rows_t<F, Op::Max, true>(in, out, rows, n, stream)
                         : launch_rows_t<F, Op::Max, false>(in, out, rows, n, stream);
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
