// Device-wide reduction: out[0] = op over in[0..n), the identity for n == 0
// ("Algorithms" page, Quadrants user guide: section
// qd.algorithms.reduce_{add,min,max} for the contract and the identities;
// "Tile operations and reductions", section "Seed versus identity", for the
// empty case: an empty fiber returns the seed).
//
// Two launches on the caller's stream, with no atomics, flags or look-back:
//  1. reduce_partials_kernel: G workgroups of four waves.  The 16-byte
//     vectors of the aligned window are cut into runs of 64*L vectors (one
//     run = L loads per lane, each load instruction covering 1 KiB), and the
//     runs into 4*G contiguous ranges, one per wave, in wave order.  Each wave
//     reduces its range; the workgroup combines its four wave totals in wave
//     order and writes one partial to scratch[b].
//  2. reduce_final_kernel: one wave combines the G partials in block order
//     and writes out[0].
// The input is read once; scratch traffic is G values.
//
// Order.  Every combine keeps the earlier operand on the left.  For integer
// add/min/max (equal values are the same bits) and floating add (order only
// changes rounding) the lanes accumulate their elements across loads and
// runs and the wave is reduced once at the end.  Floating min/max must return
// the later of two equal values (+0 vs -0) exactly as the sequential fold
// does, so there each load is reduced across the wave in lane order with the
// DPP scan before it joins the wave's running total: the grouping then never
// changes the order of the elements.
#include "device.hpp"
#include "launch.hpp"

namespace sca {

constexpr int kRedWaves = 4;          // waves per workgroup of the first launch
// 16-byte loads per lane per run, measured on MI355X (us for i32 add 2^28 /
// f32 add 2^27 / i64 max 2^26 / f32 min 2^27): 16 loads 159 / 85 / 85 / 94,
// 8 loads 174 / 88 / 88 / 92, 4 loads 174 / 91 / 93 / 96, 24 loads 165 / 85 /
// 90 / 92, 32 loads 162 / 85 / 84 / 92.  The ordered floating min/max, which
// scan every load across the wave, keep 8.
constexpr int kRedLoadsMin = 8;       // the smaller run: the most workgroups, for scratch sizing
template <class W, Op O>
constexpr bool red_ordered() {
  return (O == Op::Min || O == Op::Max) && (std::is_same_v<W, float> || std::is_same_v<W, double>);
}
template <class W, Op O>
constexpr int red_loads() { return red_ordered<W, O>() ? 8 : 16; }
// Workgroups of the first launch at most (eight per compute unit of MI355X);
// the final wave then combines at most this many partials.
constexpr int64_t kRedMaxBlocks = 2048;

template <class F, Op O, int E, int L>
__global__ __launch_bounds__(64 * kRedWaves) void reduce_partials_kernel(
    uintptr_t in_base, int64_t n_cap, const int32_t* n_dev, int64_t ph, int64_t runs_per_wave,
    uintptr_t partials) {
  using S = typename F::S;
  using W = typename F::W;
  using IO = VecIO<S, E>;
  constexpr int64_t VB = (int64_t)E * sizeof(S);
  constexpr bool kOrdered = red_ordered<W, O>();
  constexpr int64_t kRedRunVecs = (int64_t)kWave * L;
  __shared__ W s_wave[kRedWaves];

  const int lane = lane_id(), wave = wave_id();
  const W id = identity<O, W>();
  const int64_t n = live_count(n_cap, n_dev);
  const int64_t lo = ph, hi = n + ph, v_last = (hi - 1) / E;
  const int64_t runs = n == 0 ? 0 : v_last / kRedRunVecs + 1;   // runs holding live elements
  const int64_t gw = (int64_t)blockIdx.x * kRedWaves + wave;
  const int64_t r0 = gw * runs_per_wave;
  const int64_t r1 = (r0 + runs_per_wave < runs) ? r0 + runs_per_wave : runs;

  W acc = id;  // per lane (unordered ops) or wave-uniform running total (ordered)
  for (int64_t r = r0; r < r1; ++r) {
    const int64_t first = r * kRedRunVecs;
    const int64_t left = v_last + 1 - first;
    const int64_t nv = left < kRedRunVecs ? left : kRedRunVecs;
    const Buf buf(in_base + first * VB, nv * VB);
    typename IO::Raw raw[L];
#pragma unroll
    for (int j = 0; j < L; ++j) raw[j] = IO::load(buf, (uint32_t)((j * kWave + lane) * VB));
#pragma unroll
    for (int j = 0; j < L; ++j) {
      const int64_t jv = first + j * kWave;
      W x[E];
      if (jv * E >= lo && (jv + kWave) * E <= hi) {    // wave-uniform: all vectors full
        IO::template unpack<F>(raw[j], x);
      } else {
        IO::template unpack_masked<F>(raw[j], (jv + lane) * E, lo, hi, id, x);
      }
      W t = x[0];
#pragma unroll
      for (int k = 1; k < E; ++k) t = combine<O>(t, x[k]);
      if constexpr (kOrdered) {
        acc = combine<O>(acc, readlane(wave_scan_incl<O>(t), kWave - 1));
      } else {
        acc = combine<O>(acc, t);
      }
    }
  }
  if constexpr (!kOrdered) acc = readlane(wave_scan_incl<O>(acc), kWave - 1);
  if (lane == 0) s_wave[wave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    W b = s_wave[0];
#pragma unroll
    for (int w = 1; w < kRedWaves; ++w) b = combine<O>(b, s_wave[w]);
    *gptr<W>(partials + (uintptr_t)blockIdx.x * sizeof(W)) = b;
  }
}

// One wave: lane l combines partials [l*c, (l+1)*c) in order, then the lanes
// are combined in lane order.  With nparts == 0 it writes the identity.
template <class F, Op O>
__global__ __launch_bounds__(64) void reduce_final_kernel(uintptr_t partials, int64_t nparts,
                                                          uintptr_t out) {
  using W = typename F::W;
  const int lane = lane_id();
  const int64_t c = (nparts + kWave - 1) / kWave;
  W acc = identity<O, W>();
  for (int64_t i = lane * c; i < (lane + 1) * c && i < nparts; ++i)
    acc = combine<O>(acc, *gptr<W>(partials + (uintptr_t)i * sizeof(W)));
  acc = readlane(wave_scan_incl<O>(acc), kWave - 1);
  if (lane == 0) *gptr<typename F::S>(out) = narrow<F>(acc);
}

// Launch geometry for n elements at pointer phase ph (elements past the
// 128-byte line boundary before the array: the window starts on the line, so
// that every load instruction covers whole lines).  Never more workgroups than
// min(ceil(runs / 4), kRedMaxBlocks), which grows with runs; the scratch size
// takes that bound at the largest phase, which never needs fewer runs.
struct RedGeom {
  int64_t runs = 0, runs_per_wave = 0, blocks = 0;
};

static RedGeom red_geom(int64_t n, int e, int64_t ph, int64_t run_vecs) {
  RedGeom g;
  if (n <= 0) return g;
  const int64_t v_last = (n + ph - 1) / e;
  g.runs = v_last / run_vecs + 1;
  const int64_t waves_wanted = g.runs;              // at least one run per wave
  int64_t blocks = (waves_wanted + kRedWaves - 1) / kRedWaves;
  if (blocks > kRedMaxBlocks) blocks = kRedMaxBlocks;
  const int64_t waves = blocks * kRedWaves;
  g.runs_per_wave = (g.runs + waves - 1) / waves;
  // drop workgroups that would get no run at all
  const int64_t waves_used = (g.runs + g.runs_per_wave - 1) / g.runs_per_wave;
  g.blocks = (waves_used + kRedWaves - 1) / kRedWaves;
  return g;
}

static int fmt_size(Fmt f) {
  switch (f) {
    case Fmt::F16: case Fmt::BF16: return 2;
    case Fmt::F64: case Fmt::I64: case Fmt::U64: return 8;
    default: return 4;
  }
}

size_t reduce_partials(int64_t n, Fmt fmt) {
  const int e = 16 / fmt_size(fmt);
  const int64_t runs =
      red_geom(n, e, 128 / fmt_size(fmt) - 1, (int64_t)kWave * kRedLoadsMin).runs;
  const int64_t bound = (runs + kRedWaves - 1) / kRedWaves;
  return (size_t)(bound < kRedMaxBlocks ? bound : kRedMaxBlocks);
}

template <class F, Op O>
static hipError_t launch_red_t(const void* in, void* out, int64_t n, void* scratch,
                               hipStream_t stream, const int32_t* n_dev) {
  using S = typename F::S;
  constexpr int EV = 16 / (int)sizeof(S);
  const uintptr_t ia = (uintptr_t)in;
  // the window starts on the 128-byte line that holds the first element (the
  // elements before the array are read within that line, so within its page,
  // and masked as the identity)
  const int64_t ph = (int64_t)((ia % 128) / sizeof(S));
  constexpr int L = red_loads<typename F::W, O>();
  static_assert(L >= kRedLoadsMin, "scratch is sized for the smallest run");
  const RedGeom g = red_geom(n, EV, ph, (int64_t)kWave * L);
  if (g.blocks > 0) {
    reduce_partials_kernel<F, O, EV, L><<<dim3((unsigned)g.blocks), dim3(64 * kRedWaves), 0, stream>>>(
        ia - (uintptr_t)ph * sizeof(S), n, n_dev, ph, g.runs_per_wave, (uintptr_t)scratch);
  }
  reduce_final_kernel<F, O><<<dim3(1), dim3(64), 0, stream>>>((uintptr_t)scratch, g.blocks,
                                                             (uintptr_t)out);
  return hipGetLastError();
}

template <class F>
static hipError_t launch_red_f(const void* in, void* out, int64_t n, int op, void* scratch,
                               hipStream_t stream, const int32_t* n_dev) {
  switch (op) {
    case 0: return launch_red_t<F, Op::Add>(in, out, n, scratch, stream, n_dev);
    case 1: return launch_red_t<F, Op::Min>(in, out, n, scratch, stream, n_dev);
    default: return launch_red_t<F, Op::Max>(in, out, n, scratch, stream, n_dev);
  }
}

hipError_t launch_reduce(const void* in, void* out, int64_t n, Fmt fmt, int op, void* scratch,
                         hipStream_t stream, const int32_t* n_dev) {
  switch (fmt) {
    case Fmt::I32: return launch_red_f<FmtI32>(in, out, n, op, scratch, stream, n_dev);
    case Fmt::U32: return launch_red_f<FmtU32>(in, out, n, op, scratch, stream, n_dev);
    case Fmt::F32: return launch_red_f<FmtF32>(in, out, n, op, scratch, stream, n_dev);
    case Fmt::I64: return launch_red_f<FmtI64>(in, out, n, op, scratch, stream, n_dev);
    case Fmt::U64: return launch_red_f<FmtU64>(in, out, n, op, scratch, stream, n_dev);
    case Fmt::F64: return launch_red_f<FmtF64>(in, out, n, op, scratch, stream, n_dev);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sca
