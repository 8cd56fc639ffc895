// Device-wide exclusive scan (add/min/max) in one pass over the data
// ("Algorithms" page, Quadrants user guide: section
// qd.algorithms.exclusive_scan_{add,min,max} for the contract, "Related" for
// decoupled look-back as the alternative to a phase-per-launch staircase),
// and its inclusive form (out[i] = op over in[0..i], the in-place prefix sum
// of that page's PrefixSumExecutor section, here out of place and for every
// dtype and op): the same kernel with a different store stage.
//
// Workgroup b owns tile b: data waves that load, scan and store it, and one
// look-back wave.  Two tile layouts, chosen per operation (launcher below):
//  - side by side (scan_device_kernel): 8 data waves x 16 loads; load j of
//    lane l in wave w is vector (j*8 + w)*64 + l of the tile, so load round j
//    of all data waves reads one aligned 8 KiB stretch.  Each wave scans every
//    vector lane-serially and the 64 lane totals with a DPP wave scan, and
//    posts each load's total to an LDS table (load q = j*8 + w at slot q);
//    the last data wave to post scans the table (two slots per lane), which
//    gives every load the combine of the loads before it and the tile's
//    aggregate, and publishes the aggregate at once.
//  - runs (scan_device_runs_kernel): 11 data waves x 12 loads; each data wave
//    loads its own run of 64*12 vectors (load j of lane l is vector j*64 + l
//    of the run), scans it with a running carry, and posts its wave total;
//    the last data wave to post publishes the tile's aggregate.  More data
//    waves per CU hide the longer dependent chains of a compare-and-select
//    combine.
// In both:
//  - The look-back wave starts walking back over the predecessors'
//    descriptors as soon as the workgroup starts, while the data is still in
//    flight: the walk needs nothing from this tile.  When the walk ends and
//    the aggregate is out, it publishes the tile's inclusive prefix and hands
//    the exclusive prefix to the data waves through LDS.
//  - The data waves then combine tile prefix, what precedes their load or run
//    in the tile and earlier elements of the vector, and store.
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

// Scratch is sized for tiles of at least this many vectors (the launch
// shapes below have 8 x 16 x 64 = 8192 and 11 x 12 x 64 = 8448).
constexpr int64_t kDevMinTileVecs = 7168;

template <class F, Op O, bool INCL, int E, int WD, int K>
__global__ __launch_bounds__(64 * (WD + 1)) void scan_device_kernel(
    uintptr_t in_base, uintptr_t out_base, int64_t n_cap, const int32_t* n_dev, int64_t ph,
    uint64_t* desc) {
  using S = typename F::S;
  using W = typename F::W;
  using IO = VecIO<S, E>;
  constexpr int64_t VB = (int64_t)E * sizeof(S);       // bytes per vector
  constexpr int kQ = WD * K;                           // loads per tile
  constexpr int64_t kTileVecs = (int64_t)kWave * kQ;
  static_assert(kTileVecs >= kDevMinTileVecs, "scratch is sized for the smallest tile");
  static_assert(kQ == 2 * kWave, "the table of load totals is two slots per lane");
  __shared__ W s_tot[kQ];         // total of load q
  __shared__ W s_pre[kQ];         // combine of loads 0 .. q-1
  __shared__ W s_agg;             // the tile's aggregate
  __shared__ W s_prefix;          // the tile's exclusive prefix
  __shared__ uint32_t s_posted;   // data waves whose totals are in s_tot
  __shared__ uint32_t s_agg_done; // s_pre and s_agg are written, the aggregate is published

  const int lane = lane_id(), wave = wave_id();
  const int64_t tile = blockIdx.x;
  const W id = identity<O, W>();
  const int64_t n = live_count(n_cap, n_dev);
  const int64_t lo = ph, hi = n + ph, v_last = (hi - 1) / E;
  const int64_t tb = tile * kTileVecs;                 // the tile's first vector
  if (n == 0 || tb > v_last) return;                   // past the live count: nothing to do
  if (threadIdx.x == 0) {
    s_posted = 0u;
    s_agg_done = 0u;
  }
  __syncthreads();

  // Tile t's input, bounded at its last valid vector (zero bits past v_last).
  auto tile_buf = [&](int64_t t) {
    const int64_t left = v_last + 1 - t * kTileVecs;
    const int64_t nv = left <= 0 ? 0 : (left < kTileVecs ? left : kTileVecs);
    return Buf(in_base + t * kTileVecs * VB, nv * VB);
  };
  // Elements of a load whose first vector is jv, with the identity outside [lo, hi).
  auto unpack = [&](int64_t jv, const typename IO::Raw& r, W (&x)[E]) {
    if (jv * E >= lo && (jv + kWave) * E <= hi) {       // wave-uniform: all vectors full
      IO::template unpack<F>(r, x);
    } else {
      IO::template unpack_masked<F>(r, (jv + lane) * E, lo, hi, id, x);
    }
  };
  // Lane-serial scan of a load's vectors, then the wave scan of the lane
  // totals; returns the inclusive wave scan.
  auto scan_load = [&](W (&x)[E]) -> W {
#pragma unroll
    for (int k = 1; k < E; ++k) x[k] = combine<O>(x[k - 1], x[k]);
    return wave_scan_incl<O>(x[E - 1]);
  };
  // Scan of the table of load totals in load order, lane l holding loads 2l
  // and 2l+1; returns the inclusive scan of the pairs (lane 63: the tile's
  // aggregate).  The fallback below reduces a tile with this same grouping.
  auto scan_pairs = [&](W a, W b) -> W { return wave_scan_incl<O>(combine<O>(a, b)); };

  if (wave < WD) {
    // ---- data wave ----
    const Buf buf = tile_buf(tile);
    typename IO::Raw raw[K];
#pragma unroll
    for (int j = 0; j < K; ++j)
      raw[j] = IO::load(buf, (uint32_t)(((j * WD + wave) * kWave + lane) * VB));
    // x[j][k] ends as the combine of load j's elements before element k of
    // the lane's vector (exclusive) or up to it (inclusive), computed in place
    // so that only the tile's own data stays live across the barrier; lane j
    // collects load j's total
    W x[K][E];
    W tot = id;
#pragma unroll
    for (int j = 0; j < K; ++j) {
      unpack(tb + (j * WD + wave) * kWave, raw[j], x[j]);
      const W incl = scan_load(x[j]);
      const W pre = wave_shift_excl<O>(incl);
      const W t = readlane(incl, kWave - 1);
      if (lane == j) tot = t;
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
    if (lane < K) s_tot[lane * WD + wave] = tot;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    uint32_t before = 0;
    if (lane == 0)
      before = __hip_atomic_fetch_add(&s_posted, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
    before = __builtin_amdgcn_readfirstlane(before);
    if (before == (uint32_t)WD - 1) {
      // the last data wave to post: every load total is in the table
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      const W a = s_tot[2 * lane], b = s_tot[2 * lane + 1];
      const W sp = scan_pairs(a, b);
      const W e = wave_shift_excl<O>(sp);
      s_pre[2 * lane] = e;
      s_pre[2 * lane + 1] = combine<O>(e, a);
      const W agg = readlane(sp, kWave - 1);
      if (lane == 0) {
        s_agg = agg;
        if (tile > 0) Desc<W>::publish(desc, tile, kAgg, agg);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      if (lane == 0)
        __hip_atomic_store(&s_agg_done, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    __syncthreads();  // sleeps in hardware until the look-back wave has the prefix
    const W tp = s_prefix;
    if (tb * E >= lo && (tb + kTileVecs) * E <= hi) {   // tile-uniform: all vectors full
      // one buffer per load, so every store takes the lane's offset alone
#pragma unroll
      for (int j = 0; j < K; ++j) {
        const int q = j * WD + wave;
        const W p = combine<O>(tp, s_pre[q]);
        const Buf ob(out_base + (tb + q * kWave) * VB, kWave * VB);
        W y[E];
#pragma unroll
        for (int k = 0; k < E; ++k) y[k] = combine<O>(p, x[j][k]);
        IO::template store_full<F>(ob, (uint32_t)(lane * VB), y);
      }
    } else {
#pragma unroll
      for (int j = 0; j < K; ++j) {
        const int q = j * WD + wave;
        const W p = combine<O>(tp, s_pre[q]);
        W y[E];
#pragma unroll
        for (int k = 0; k < E; ++k) y[k] = combine<O>(p, x[j][k]);
        const int64_t v = tb + q * kWave + lane;
        if (v <= v_last) IO::template store<F>(out_base, v, lo, hi, y);
      }
    }
  } else {
    // ---- look-back wave ----
    W prefix = id;
    if (tile > 0) {
      // fallback for a late predecessor: reduce its input with the grouping
      // its own data waves use (each load scanned alone, then the table of
      // load totals scanned in pairs), so the result is bit for bit the
      // aggregate that tile would publish, floating add included; a few loads
      // at a time (this rare path must not raise the kernel's register count,
      // which sets how many workgroups fit on a CU)
      auto reduce_tile = [&](int64_t t) -> W {
        constexpr int kG = 4;
        static_assert(kQ % kG == 0, "whole groups of loads");
        const Buf buf = tile_buf(t);
        W a = id, b = id;   // lane l: totals of loads 2l and 2l+1
#pragma unroll 1
        for (int g = 0; g < kQ / kG; ++g) {
          typename IO::Raw r[kG];
#pragma unroll
          for (int i = 0; i < kG; ++i)
            r[i] = IO::load(buf, (uint32_t)(((g * kG + i) * kWave + lane) * VB));
#pragma unroll
          for (int i = 0; i < kG; ++i) {
            const int q = g * kG + i;
            W y[E];
            unpack(t * kTileVecs + q * kWave, r[i], y);
            const W tq = readlane(scan_load(y), kWave - 1);
            if (lane == (q >> 1)) {
              if (i & 1) b = tq;
              else a = tq;
            }
          }
        }
        return readlane(scan_pairs(a, b), kWave - 1);
      };
      prefix = look_back<O, W, kPollLong>(desc, tile, kLookBackTimeout, reduce_tile);
    }
    while (!lds_flag_set(&s_agg_done)) __builtin_amdgcn_s_sleep(1);
    if (lane == 0) {
      Desc<W>::publish(desc, tile, kInc, combine<O>(prefix, s_agg));
      s_prefix = prefix;
    }
    __syncthreads();
  }
}

// The runs layout (contiguous run of 64*K vectors per data wave).
template <class F, Op O, bool INCL, int E, int WD, int K>
__global__ __launch_bounds__(64 * (WD + 1)) void scan_device_runs_kernel(
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

// Tiles of tv vectors covering window elements [ph, n + ph) in vectors of e
// elements.
static int64_t tiles_for(int64_t n, int64_t ph, int e, int64_t tv) {
  if (n <= 0) return 0;
  const int64_t v_last = (n + ph - 1) / e;
  return v_last / tv + 1;
}

// Sized for the slowest path (one element per vector, no phase) and the
// smallest tile, so one scratch size serves every pointer alignment and launch
// shape: with vectors of e >= 2 elements and a window phase below 128 bytes,
// (n + ph - 1) / e never exceeds n - 1 by enough to need another tile.
size_t scan_device_tiles(int64_t n, Fmt fmt) {
  (void)fmt;
  return (size_t)tiles_for(n, 0, 1, kDevMinTileVecs);
}

// Tile layout by operation, measured on MI355X (us per exclusive scan; runs
// 11 x 12 against side by side 8 x 16): i32 add 2^28 367.9 / 363.3, f32 add
// 2^27 191.7 / 188.8, i64 add 2^26 198.8 / 196.0, f64 add 2^26 198.3 /
// 195.7; u32 max 2^27 190.3 / 189.1; f32 min 2^27 190.5 / 195.3, f32 max
// 2^27 190.0 / 196.3, i64 min 2^26 195.5 / 202.6, i64 max 2^26 195.7 /
// 202.0.  Side by side, a load round of the data waves covers one aligned
// 8 KiB stretch, which a copy that holds its data until a barrier moves
// faster (6.2 TB/s against 5.7 for 8 KiB runs); but it has 8 data waves per
// workgroup against 11, and a combine that is a compare and a select (min and
// max of floats, which keep the later of two equal values, and of 64-bit
// integers) makes every DPP step three instructions, which then stall the
// fewer waves.  Add takes the side-by-side tiles, min and max the runs (the
// 32-bit integer min/max tie, and side by side their inclusive forms need
// more registers than two workgroups per CU allow).
template <Op O>
constexpr bool kSideBySide = O == Op::Add;

template <class F, Op O, bool INCL>
static hipError_t launch_dev_cfg(const void* in, void* out, int64_t n, void* scratch,
                                 hipStream_t stream, const int32_t* n_dev, bool descs_clear) {
  using S = typename F::S;
  constexpr bool kSide = kSideBySide<O>;
  constexpr int WD = kSide ? 8 : 11;    // data waves (plus the look-back wave)
  constexpr int K = kSide ? 16 : 12;    // loads per lane
  constexpr int EV = 16 / (int)sizeof(S);
  constexpr int64_t TV = (int64_t)kWave * WD * K;
  const uintptr_t ia = (uintptr_t)in, oa = (uintptr_t)out;
  uint64_t* desc = desc_base(scratch);
  const bool vec = (ia % 16) == (oa % 16);
  const int e = vec ? EV : 1;
  // The window starts on the 16-byte vector that holds the first element, or,
  // when input and output share their place in a 128-byte line, on that
  // line, so that every load and store instruction covers whole lines (one
  // that starts mid-line touches nine lines per KiB instead of eight).  The
  // window elements before the array are read (within the array's first line,
  // so within its page) and masked as the identity; none is stored.
  const bool line = (ia % 128) == (oa % 128);
  const int64_t ph = vec ? (int64_t)((ia % (line ? 128 : 16)) / sizeof(S)) : 0;
  const int64_t ntiles = tiles_for(n, ph, e, TV);
  if (!descs_clear) {
    const hipError_t err = launch_fill_desc(desc, ntiles, Desc<typename F::W>::kWords, stream);
    if (err != hipSuccess) return err;
  }
  const dim3 grid((unsigned)ntiles), block(64 * (WD + 1));
  const uintptr_t ib = vec ? ia - ph * sizeof(S) : ia, ob = vec ? oa - ph * sizeof(S) : oa;
  if constexpr (kSide) {
    if (vec)
      scan_device_kernel<F, O, INCL, EV, WD, K><<<grid, block, 0, stream>>>(ib, ob, n, n_dev, ph, desc);
    else
      scan_device_kernel<F, O, INCL, 1, WD, K><<<grid, block, 0, stream>>>(ib, ob, n, n_dev, 0, desc);
  } else {
    if (vec)
      scan_device_runs_kernel<F, O, INCL, EV, WD, K><<<grid, block, 0, stream>>>(ib, ob, n, n_dev, ph,
                                                                               desc);
    else
      scan_device_runs_kernel<F, O, INCL, 1, WD, K><<<grid, block, 0, stream>>>(ib, ob, n, n_dev, 0,
                                                                              desc);
  }
  return hipGetLastError();
}

template <class F, Op O>
static hipError_t launch_dev_t(const void* in, void* out, int64_t n, bool incl, void* scratch,
                               hipStream_t stream, const int32_t* n_dev, bool descs_clear) {
  return incl ? launch_dev_cfg<F, O, true>(in, out, n, scratch, stream, n_dev, descs_clear)
              : launch_dev_cfg<F, O, false>(in, out, n, scratch, stream, n_dev, descs_clear);
}

template <class F>
static hipError_t launch_dev_f(const void* in, void* out, int64_t n, int op, bool incl,
                               void* scratch, hipStream_t stream, const int32_t* n_dev,
                               bool descs_clear) {
  switch (op) {
    case 0: return launch_dev_t<F, Op::Add>(in, out, n, incl, scratch, stream, n_dev, descs_clear);
    case 1: return launch_dev_t<F, Op::Min>(in, out, n, incl, scratch, stream, n_dev, descs_clear);
    default: return launch_dev_t<F, Op::Max>(in, out, n, incl, scratch, stream, n_dev, descs_clear);
  }
}

hipError_t launch_scan_device(const void* in, void* out, int64_t n, Fmt fmt, int op,
                              bool inclusive, void* scratch, hipStream_t stream,
                              const int32_t* n_dev, bool descs_clear) {
  switch (fmt) {
    case Fmt::I32: return launch_dev_f<FmtI32>(in, out, n, op, inclusive, scratch, stream, n_dev, descs_clear);
    case Fmt::U32: return launch_dev_f<FmtU32>(in, out, n, op, inclusive, scratch, stream, n_dev, descs_clear);
    case Fmt::F32: return launch_dev_f<FmtF32>(in, out, n, op, inclusive, scratch, stream, n_dev, descs_clear);
    case Fmt::I64: return launch_dev_f<FmtI64>(in, out, n, op, inclusive, scratch, stream, n_dev, descs_clear);
    case Fmt::U64: return launch_dev_f<FmtU64>(in, out, n, op, inclusive, scratch, stream, n_dev, descs_clear);
    case Fmt::F64: return launch_dev_f<FmtF64>(in, out, n, op, inclusive, scratch, stream, n_dev, descs_clear);
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
