// Device-wide exclusive scan (add/min/max) in one pass over the data
// ("Algorithms" page, Quadrants user guide: section
// qd.algorithms.exclusive_scan_{add,min,max} for the contract, "Related" for
// decoupled look-back as the alternative to a phase-per-launch staircase).
//
// Workgroup b owns tile b (WPB waves, K 16-byte vectors per lane).  It loads
// its tile (load j of lane l in wave w is vector (w*K + j)*64 + l of the
// tile, so every load instruction covers 1 KiB of contiguous memory) and:
//   1. scans every vector lane-serially, then the 64 lane totals with a DPP
//      wave scan, keeping per vector the combine of everything before it in
//      the wave;
//   2. publishes the wave totals through LDS; wave 0 forms the tile
//      aggregate, publishes it, looks back over predecessor descriptors to
//      get the tile's exclusive prefix, and publishes its inclusive prefix;
//   3. after one more barrier every lane combines tile prefix, earlier waves,
//      earlier vectors and earlier elements of its vector, and stores.
// The input is read once and the output written once.  Tile ids are the
// workgroup ids: no atomic counter (a device-wide atomic on one address
// serializes at about 11 ns per tile on MI355X); the look-back's bounded wait
// (device.hpp) keeps this correct and deadlock-free under any workgroup order.
#include "device.hpp"
#include "launch.hpp"

namespace sca {

// Smallest tile (in vectors) of any launch shape below; scratch is sized for it.
constexpr int64_t kDevMinTileVecs = 1024;

template <class F, Op O, int E, int WPB, int K>
__global__ __launch_bounds__(64 * WPB) void scan_device_kernel(uintptr_t in_base, uintptr_t out_base,
                                                              int64_t n, int64_t ph, int64_t ntiles,
                                                              uint64_t* desc) {
  using S = typename F::S;
  using W = typename F::W;
  using IO = VecIO<S, E>;
  constexpr int64_t VB = (int64_t)E * sizeof(S);       // bytes per vector
  constexpr int64_t kWaveVecs = (int64_t)kWave * K;
  constexpr int64_t kTileVecs = kWaveVecs * WPB;
  static_assert(kTileVecs >= kDevMinTileVecs, "scratch is sized for the smallest tile");
  __shared__ W s_wave[WPB];
  __shared__ W s_prefix;

  const int lane = lane_id(), wave = wave_id();
  const int64_t tile = blockIdx.x;
  const W id = identity<O, W>();
  const int64_t lo = ph, hi = n + ph, v_last = (hi - 1) / E;

  // A wave's K loads of the run of 64*K vectors starting at `first` (zero bits past v_last).
  auto load = [&](int64_t first, typename IO::Raw (&raw)[K]) {
    const int64_t left = v_last + 1 - first;
    const int64_t nv = left <= 0 ? 0 : (left < kWaveVecs ? left : kWaveVecs);
    const Buf buf(in_base + first * VB, nv * VB);
#pragma unroll
    for (int j = 0; j < K; ++j) raw[j] = IO::load(buf, (uint32_t)((j * kWave + lane) * VB));
  };
  // Elements of load j (first vector of the load: jv) with the identity outside [lo, hi).
  auto unpack = [&](int64_t jv, const typename IO::Raw& r, W (&x)[E]) {
    if (jv * E >= lo && (jv + kWave) * E <= hi) {       // wave-uniform: all vectors full
      IO::template unpack<F>(r, x);
    } else {
      IO::template unpack_masked<F>(r, (jv + lane) * E, lo, hi, id, x);
    }
  };

  const int64_t wb = tile * kTileVecs + wave * kWaveVecs;  // this wave's first vector
  typename IO::Raw raw[K];
  load(wb, raw);

  // 1. within the wave
  W x[K][E];
  W pre[K];
  W carry = id;
#pragma unroll
  for (int j = 0; j < K; ++j) {
    unpack(wb + j * kWave, raw[j], x[j]);
#pragma unroll
    for (int k = 1; k < E; ++k) x[j][k] = combine<O>(x[j][k - 1], x[j][k]);
    const W incl = wave_scan_incl<O>(x[j][E - 1]);
    pre[j] = combine<O>(carry, wave_shift_excl<O>(incl));
    carry = combine<O>(carry, readlane(incl, kWave - 1));
  }
  if (lane == 0) s_wave[wave] = carry;
  __syncthreads();

  // 2. across tiles
  if (wave == 0) {
    W agg = s_wave[0];
#pragma unroll
    for (int w = 1; w < WPB; ++w) agg = combine<O>(agg, s_wave[w]);
    W prefix = id;
    if (tile == 0) {
      if (lane == 0) Desc<W>::publish(desc, tile, kInc, agg);
    } else {
      if (lane == 0) Desc<W>::publish(desc, tile, kAgg, agg);
      // fallback for a late predecessor: reduce its input in element order
      auto reduce_tile = [&](int64_t t) -> W {
        W acc = id;
        for (int c = 0; c < WPB; ++c) {
          typename IO::Raw r[K];
          const int64_t first = t * kTileVecs + c * kWaveVecs;
          load(first, r);
#pragma unroll
          for (int j = 0; j < K; ++j) {
            W y[E];
            unpack(first + j * kWave, r[j], y);
#pragma unroll
            for (int k = 1; k < E; ++k) y[k] = combine<O>(y[k - 1], y[k]);
            acc = combine<O>(acc, readlane(wave_scan_incl<O>(y[E - 1]), kWave - 1));
          }
        }
        return acc;
      };
      prefix = look_back<O, W>(desc, tile, kLookBackTimeout, reduce_tile);
      if (lane == 0) Desc<W>::publish(desc, tile, kInc, combine<O>(prefix, agg));
    }
    if (lane == 0) s_prefix = prefix;
  }
  __syncthreads();

  // 3. outputs
  W wp = s_prefix;
  for (int w = 0; w < wave; ++w) wp = combine<O>(wp, s_wave[w]);
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const W q = combine<O>(wp, pre[j]);
    W y[E];
    y[0] = q;
#pragma unroll
    for (int k = 1; k < E; ++k) y[k] = combine<O>(q, x[j][k - 1]);
    const int64_t v = wb + j * kWave + lane;
    if (v <= v_last) IO::template store<F>(out_base, v, lo, hi, y);
  }
}

// Tiles of tv vectors covering window elements [ph, n + ph) (ph < e) in
// vectors of e elements.
static int64_t tiles_for(int64_t n, int e, int64_t tv) {
  if (n <= 0) return 0;
  const int64_t v_last = (n - 1 + (e - 1)) / e;
  return v_last / tv + 1;
}

static int fmt_bytes(Fmt f) {
  switch (f) {
    case Fmt::F16: case Fmt::BF16: return 2;
    case Fmt::F64: case Fmt::I64: case Fmt::U64: return 8;
    default: return 4;
  }
}

size_t scan_device_desc_words(Fmt fmt) { return fmt_bytes(fmt) == 8 ? 4 : 1; }

// Sized for the slowest path (one element per vector) and the smallest tile,
// so one scratch size serves every pointer alignment and launch shape.
size_t scan_device_tiles(int64_t n, Fmt fmt) {
  (void)fmt;
  return (size_t)tiles_for(n, 1, kDevMinTileVecs);
}

// One launch shape: WPB waves per workgroup, K vectors per lane per tile.
template <class F, Op O, int WPB, int K>
static hipError_t launch_dev_cfg(const void* in, void* out, int64_t n, void* scratch,
                                 hipStream_t stream) {
  using S = typename F::S;
  constexpr int EV = 16 / (int)sizeof(S);
  constexpr int64_t TV = (int64_t)kWave * WPB * K;
  const uintptr_t ia = (uintptr_t)in, oa = (uintptr_t)out;
  uint64_t* desc = (uint64_t*)scratch;
  const bool vec = (ia % 16) == (oa % 16);
  const int e = vec ? EV : 1;
  const int64_t ph = vec ? (int64_t)((ia % 16) / sizeof(S)) : 0;
  const int64_t ntiles = tiles_for(n, e, TV);
  hipError_t err = launch_fill_zero(scratch, (size_t)ntiles * Desc<typename F::W>::kWords * 8,
                                    stream);
  if (err != hipSuccess) return err;
  const dim3 grid((unsigned)ntiles), block(64 * WPB);
  if (vec) {
    scan_device_kernel<F, O, EV, WPB, K><<<grid, block, 0, stream>>>(
        ia - ph * sizeof(S), oa - ph * sizeof(S), n, ph, ntiles, desc);
  } else {
    scan_device_kernel<F, O, 1, WPB, K><<<grid, block, 0, stream>>>(ia, oa, n, 0, ntiles, desc);
  }
  return hipGetLastError();
}

// Launch shape measured on MI355X over 2^28 32-bit elements: four waves of
// sixteen loads (64 KiB tiles) beat both wider workgroups and smaller tiles;
// smaller tiles spend longer in look-back than they gain in occupancy.
template <class F, Op O>
static hipError_t launch_dev_t(const void* in, void* out, int64_t n, void* scratch,
                               hipStream_t stream) {
  return launch_dev_cfg<F, O, 4, 16>(in, out, n, scratch, stream);
}

template <class F>
static hipError_t launch_dev_f(const void* in, void* out, int64_t n, int op, void* scratch,
                               hipStream_t stream) {
  switch (op) {
    case 0: return launch_dev_t<F, Op::Add>(in, out, n, scratch, stream);
    case 1: return launch_dev_t<F, Op::Min>(in, out, n, scratch, stream);
    default: return launch_dev_t<F, Op::Max>(in, out, n, scratch, stream);
  }
}

hipError_t launch_scan_device(const void* in, void* out, int64_t n, Fmt fmt, int op, void* scratch,
                              hipStream_t stream) {
  switch (fmt) {
    case Fmt::I32: return launch_dev_f<FmtI32>(in, out, n, op, scratch, stream);
    case Fmt::U32: return launch_dev_f<FmtU32>(in, out, n, op, scratch, stream);
    case Fmt::F32: return launch_dev_f<FmtF32>(in, out, n, op, scratch, stream);
    case Fmt::I64: return launch_dev_f<FmtI64>(in, out, n, op, scratch, stream);
    case Fmt::U64: return launch_dev_f<FmtU64>(in, out, n, op, scratch, stream);
    case Fmt::F64: return launch_dev_f<FmtF64>(in, out, n, op, scratch, stream);
    default: return hipErrorInvalidValue;
  }
}

// ---------------------------------------------------------------------------
// Small fill kernel used to reset scratch at the start of each call.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void fill_zero_kernel(uint4* p, int64_t n16) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = uint4{0u, 0u, 0u, 0u};
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t stream) {
  const int64_t n16 = (int64_t)((bytes + 15) / 16);
  if (n16 == 0) return hipSuccess;
  int64_t blocks = (n16 + kBlock - 1) / kBlock;
  if (blocks > 2048) blocks = 2048;
  fill_zero_kernel<<<dim3((unsigned)blocks), dim3(kBlock), 0, stream>>>((uint4*)p, n16);
  return hipGetLastError();
}

}  // namespace sca
