// Device-wide exclusive scan (add/min/max) in one pass over the data
// ("Algorithms" page, Quadrants user guide: section
// qd.algorithms.exclusive_scan_{add,min,max} for the contract, "Related" for
// decoupled look-back as the alternative to a phase-per-launch staircase),
// and its inclusive form (out[i] = op over in[0..i], the in-place prefix sum
// of that page's PrefixSumExecutor section, here out of place and for every
// dtype and op): the same kernel with a different store stage.
//
// Workgroup b owns tile b.  It has WD data waves and one look-back wave.
//  - Each data wave loads its run of 64*K 16-byte vectors (load j of lane l
//    is vector j*64 + l of the run, so every load instruction covers 1 KiB),
//    scans every vector lane-serially and the 64 lane totals with a DPP wave
//    scan, and posts its wave total to LDS; the last data wave to post
//    publishes the tile's aggregate at once.
//  - The look-back wave starts walking back over the predecessors'
//    descriptors as soon as the workgroup starts, while the data is still in
//    flight: the walk needs nothing from this tile.  When the walk ends and
//    the aggregate is out, it publishes the tile's inclusive prefix and hands
//    the exclusive prefix to the data waves through LDS.
//  - The data waves then combine tile prefix, earlier waves, earlier vectors
//    and earlier elements of the vector, and store.
// The input is read once and the output written once.  Tile ids are the
// workgroup ids: no atomic counter (a device-wide atomic on one address
// serializes at about 11 ns per tile on MI355X); the look-back's bounded wait
// (device.hpp) keeps this correct and deadlock-free under any workgroup order.
// The waves meet through an LDS counter and flag (no barrier), so the
// look-back never holds up the data waves' loads and scans; one barrier then
// hands the prefix back, with the data waves asleep in it.
#include <atomic>
#include <mutex>

#include "device.hpp"
#include "launch.hpp"

// Scratch of the allocation-free entry point: one copy of this array per GPU,
// held until the process ends and shared by every such call on that GPU (so
// two of them in flight at once on one GPU race).  In host code the name
// `scratch` denotes a host-side stand-in, not a device address: host code
// only ever uses the address hipGetSymbolAddress returns for the current
// device (noalloc_scratch below).
static __device__ __align__(256) uint8_t scratch[sca::kNoAllocScratchBytes];

namespace sca {

// Scratch is sized for tiles of at least this many vectors (7 x 16 x 64; the
// launch shape below, 11 data waves x 12 loads x 64 lanes, has 8448).
constexpr int64_t kDevMinTileVecs = 7168;

template <class F, Op O, bool INCL, int E, int WD, int K>
__global__ __launch_bounds__(64 * (WD + 1)) void scan_device_kernel(
    uintptr_t in_base, uintptr_t out_base, int64_t n_cap, const int32_t* n_dev, int64_t ph,
    uint64_t* desc) {
  using S = typename F::S;
  using W = typename F::W;
  using IO = VecIO<S, E>;
  constexpr int64_t VB = (int64_t)E * sizeof(S);       // bytes per vector
  constexpr int64_t kWaveVecs = (int64_t)kWave * K;
  constexpr int64_t kTileVecs = kWaveVecs * WD;
  static_assert(kTileVecs >= kDevMinTileVecs, "scratch is sized for the smallest tile");
  __shared__ W s_wave[WD];
  __shared__ W s_prefix;
  __shared__ uint32_t s_posted;   // data waves whose totals are in s_wave
  __shared__ uint32_t s_agg_done; // the tile's aggregate is published

  const int lane = lane_id(), wave = wave_id();
  const int64_t tile = blockIdx.x;
  const W id = identity<O, W>();
  const int64_t n = live_count(n_cap, n_dev);
  const int64_t lo = ph, hi = n + ph, v_last = (hi - 1) / E;
  if (n == 0 || tile * kTileVecs > v_last) return;   // past the live count: nothing to do
  if (threadIdx.x == 0) {
    s_posted = 0u;
    s_agg_done = 0u;
  }
  __syncthreads();

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

  if (wave < WD) {
    // ---- data wave ----
    const int64_t wb = tile * kTileVecs + wave * kWaveVecs;  // this wave's first vector
    typename IO::Raw raw[K];
    load(wb, raw);
    // x[j][k] ends as the combine of this wave's elements before element k of
    // the lane's vector j (exclusive) or up to it (inclusive), computed in
    // place so that only the tile's own data stays live across the barrier
    W x[K][E];
    W carry = id;
#pragma unroll
    for (int j = 0; j < K; ++j) {
      unpack(wb + j * kWave, raw[j], x[j]);
#pragma unroll
      for (int k = 1; k < E; ++k) x[j][k] = combine<O>(x[j][k - 1], x[j][k]);
      const W incl = wave_scan_incl<O>(x[j][E - 1]);
      const W pre = combine<O>(carry, wave_shift_excl<O>(incl));
      carry = combine<O>(carry, readlane(incl, kWave - 1));
      if constexpr (INCL) {
#pragma unroll
        for (int k = 0; k < E; ++k) x[j][k] = combine<O>(pre, x[j][k]);
      } else {
#pragma unroll
        for (int k = E - 1; k > 0; --k) x[j][k] = combine<O>(pre, x[j][k - 1]);
        x[j][0] = pre;
      }
#pragma unroll
      for (int k = 0; k < E; ++k) materialize(x[j][k]);
    }
    if (lane == 0) post_wave_total<O, W, WD>(carry, wave, tile, s_wave, &s_posted, &s_agg_done, desc);
    __syncthreads();  // sleeps in hardware until the look-back wave has the prefix
    W wp = s_prefix;
    for (int w = 0; w < wave; ++w) wp = combine<O>(wp, s_wave[w]);
    if (wb * E >= lo && (wb + kWaveVecs) * E <= hi) {   // wave-uniform: all vectors full
      // one buffer per 4 KiB of the run, so every store takes the lane's
      // offset plus an immediate one (a single offset register)
#pragma unroll
      for (int j = 0; j < K; ++j) {
        const Buf ob(out_base + (wb + (j & ~3) * kWave) * VB, 4 * kWave * VB);
        W y[E];
#pragma unroll
        for (int k = 0; k < E; ++k) y[k] = combine<O>(wp, x[j][k]);
        IO::template store_full<F>(ob, (uint32_t)(((j & 3) * kWave + lane) * VB), y);
      }
    } else {
#pragma unroll
      for (int j = 0; j < K; ++j) {
        W y[E];
#pragma unroll
        for (int k = 0; k < E; ++k) y[k] = combine<O>(wp, x[j][k]);
        const int64_t v = wb + j * kWave + lane;
        if (v <= v_last) IO::template store<F>(out_base, v, lo, hi, y);
      }
    }
  } else {
    // ---- look-back wave ----
    auto tile_agg = [&]() {
      W a = s_wave[0];
#pragma unroll
      for (int w = 1; w < WD; ++w) a = combine<O>(a, s_wave[w]);
      return a;
    };
    W prefix = id;
    if (tile > 0) {
      // fallback for a late predecessor: reduce its input with the grouping
      // its own data waves use (each wave's K loads folded from the identity,
      // then the wave totals in wave order), so the result is bit for bit the
      // aggregate that tile would publish, floating add included; a few loads
      // at a time (this rare path must not raise the kernel's register count,
      // which sets how many workgroups fit on a CU)
      auto reduce_tile = [&](int64_t t) -> W {
        constexpr int kG = 4;
        static_assert(K % kG == 0, "a wave's run is whole groups of loads");
        const int64_t first = t * kTileVecs;
        const int64_t left = v_last + 1 - first;
        const int64_t nv = left <= 0 ? 0 : (left < kTileVecs ? left : kTileVecs);
        const Buf buf(in_base + first * VB, nv * VB);
        W acc = id;
#pragma unroll 1
        for (int w = 0; w < WD; ++w) {
          W wsum = id;
#pragma unroll 1
          for (int g = 0; g < K / kG; ++g) {
            const int j0 = w * K + g * kG;      // the tile's load index
            typename IO::Raw r[kG];
#pragma unroll
            for (int j = 0; j < kG; ++j)
              r[j] = IO::load(buf, (uint32_t)(((j0 + j) * kWave + lane) * VB));
#pragma unroll
            for (int j = 0; j < kG; ++j) {
              W y[E];
              unpack(first + (j0 + j) * kWave, r[j], y);
#pragma unroll
              for (int k = 1; k < E; ++k) y[k] = combine<O>(y[k - 1], y[k]);
              wsum = combine<O>(wsum, readlane(wave_scan_incl<O>(y[E - 1]), kWave - 1));
            }
          }
          acc = w == 0 ? wsum : combine<O>(acc, wsum);
        }
        return acc;
      };
      prefix = look_back<O, W, kPollLong>(desc, tile, kLookBackTimeout, reduce_tile);
    }
    while (!lds_flag_set(&s_agg_done)) __builtin_amdgcn_s_sleep(1);
    if (lane == 0) {
      Desc<W>::publish(desc, tile, kInc, combine<O>(prefix, tile_agg()));
      s_prefix = prefix;
    }
    __syncthreads();
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


// Sized for the slowest path (one element per vector) and the smallest tile,
// so one scratch size serves every pointer alignment and launch shape.
size_t scan_device_tiles(int64_t n, Fmt fmt) {
  (void)fmt;
  return (size_t)tiles_for(n, 1, kDevMinTileVecs);
}

// One launch shape: WD data waves (plus the look-back wave), K vectors per
// lane per tile.
template <class F, Op O, bool INCL, int WD, int K>
static hipError_t launch_dev_cfg(const void* in, void* out, int64_t n, void* scratch,
                                 hipStream_t stream, const int32_t* n_dev) {
  using S = typename F::S;
  constexpr int EV = 16 / (int)sizeof(S);
  constexpr int64_t TV = (int64_t)kWave * WD * K;
  const uintptr_t ia = (uintptr_t)in, oa = (uintptr_t)out;
  uint64_t* desc = desc_base(scratch);
  const bool vec = (ia % 16) == (oa % 16);
  const int e = vec ? EV : 1;
  const int64_t ph = vec ? (int64_t)((ia % 16) / sizeof(S)) : 0;
  const int64_t ntiles = tiles_for(n, e, TV);
  hipError_t err = launch_fill_desc(desc, ntiles, Desc<typename F::W>::kWords, stream);
  if (err != hipSuccess) return err;
  const dim3 grid((unsigned)ntiles), block(64 * (WD + 1));
  if (vec) {
    scan_device_kernel<F, O, INCL, EV, WD, K><<<grid, block, 0, stream>>>(
        ia - ph * sizeof(S), oa - ph * sizeof(S), n, n_dev, ph, desc);
  } else {
    scan_device_kernel<F, O, INCL, 1, WD, K><<<grid, block, 0, stream>>>(ia, oa, n, n_dev, 0,
                                                                        desc);
  }
  return hipGetLastError();
}

// Launch shape measured on MI355X (us per scan; i32 add over 2^28 / i64 min
// over 2^26): 11 data waves x 12 loads (132 KiB tiles) 365.8 / 208.3,
// 7 x 16: 374.2 / 215.4 (3 workgroups per CU; 368.2 when capped at 2),
// 7 x 20: 369.6, 8 x 16: 370.4 / 292.3, 15 x 8: 424.0 / 264.4.  An earlier
// sweep over 3 and 4 data waves was slower still (3 x 16: 436).  Few, large
// tiles win, since each look-back costs microseconds of latency; but more
// resident tiles per CU (a wider address window in flight) lose, so the
// shape is also chosen for two workgroups per CU.
template <class F, Op O>
static hipError_t launch_dev_t(const void* in, void* out, int64_t n, bool incl, void* scratch,
                               hipStream_t stream, const int32_t* n_dev) {
  return incl ? launch_dev_cfg<F, O, true, 11, 12>(in, out, n, scratch, stream, n_dev)
              : launch_dev_cfg<F, O, false, 11, 12>(in, out, n, scratch, stream, n_dev);
}

template <class F>
static hipError_t launch_dev_f(const void* in, void* out, int64_t n, int op, bool incl,
                               void* scratch, hipStream_t stream, const int32_t* n_dev) {
  switch (op) {
    case 0: return launch_dev_t<F, Op::Add>(in, out, n, incl, scratch, stream, n_dev);
    case 1: return launch_dev_t<F, Op::Min>(in, out, n, incl, scratch, stream, n_dev);
    default: return launch_dev_t<F, Op::Max>(in, out, n, incl, scratch, stream, n_dev);
  }
}

hipError_t launch_scan_device(const void* in, void* out, int64_t n, Fmt fmt, int op,
                              bool inclusive, void* scratch, hipStream_t stream,
                              const int32_t* n_dev) {
  switch (fmt) {
    case Fmt::I32: return launch_dev_f<FmtI32>(in, out, n, op, inclusive, scratch, stream, n_dev);
    case Fmt::U32: return launch_dev_f<FmtU32>(in, out, n, op, inclusive, scratch, stream, n_dev);
    case Fmt::F32: return launch_dev_f<FmtF32>(in, out, n, op, inclusive, scratch, stream, n_dev);
    case Fmt::I64: return launch_dev_f<FmtI64>(in, out, n, op, inclusive, scratch, stream, n_dev);
    case Fmt::U64: return launch_dev_f<FmtU64>(in, out, n, op, inclusive, scratch, stream, n_dev);
    case Fmt::F64: return launch_dev_f<FmtF64>(in, out, n, op, inclusive, scratch, stream, n_dev);
    default: return hipErrorInvalidValue;
  }
}

// Device address of the calling thread's current GPU's copy of `scratch`,
// looked up once per device (with that device current) and kept.
namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (p == nullptr) return hipErrorInvalidSymbol;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

// ---------------------------------------------------------------------------
// Small kernel that resets the used words of `ntiles` descriptors (one per
// 128-byte line) at the start of each call.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void fill_desc_kernel(uint64_t* d, int64_t ntiles, int words) {
  const int64_t total = ntiles * words;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x)
    d[(i / words) * kDescLineWords + i % words] = 0ull;
}

hipError_t launch_fill_desc(uint64_t* desc, int64_t ntiles, int words, hipStream_t stream) {
  const int64_t total = ntiles * words;
  if (total <= 0) return hipSuccess;
  int64_t blocks = (total + kBlock - 1) / kBlock;
  if (blocks > 2048) blocks = 2048;
  fill_desc_kernel<<<dim3((unsigned)blocks), dim3(kBlock), 0, stream>>>(desc, ntiles, words);
  return hipGetLastError();
}

}  // namespace sca
