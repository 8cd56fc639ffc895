// Reduce-by-key ("Algorithms" page, Quadrants user guide, section
// qd.algorithms.reduce_by_key_add): every maximal run of consecutive equal
// keys becomes one output pair (key, sum of the run's values), in input
// order, and the number of runs goes to num_runs[0].
//
// The page realizes it as head flags, an exclusive scan of the flags into an
// n-entry buffer, and a scatter that atomically adds every value into its run
// (section "Under the hood").  Here one kernel does it in a single pass, with
// no index buffer and no atomics, as a segmented scan ("Tile operations and
// reductions": a segmented scan carries a lifted (head, value) state through
// the same associative machinery):
//   - element i carries the pair (h_i, v_i), h_i = 1 when it starts a run
//     (i == 0 or key[i] differs from key[i-1]);
//   - pairs combine as (c1, s1) (+) (c2, s2) = (c1 + c2, c2 ? s2 : s1 + s2):
//     c counts the run starts in a span and s sums its values after the last
//     start.  This is associative and keeps the earlier span on the left, so
//     the DPP wave scan, the LDS exchange and the decoupled look-back of the
//     device-wide scan carry it unchanged (tile descriptors hold the 64-bit
//     pair);
//   - with the exclusive pair (c, s) of a run-starting element i, run c
//     begins at i: keys_out[c] = key[i]; and when c > 0, run c-1 ended at
//     i-1 with sum s: values_out[c-1] = s.  The element at n-1 closes the
//     last run and writes num_runs.
// Keys compare with their own type's == (an f32 NaN key never equals
// anything; +0 equals -0); each run keeps its first key.  Integer values
// wrap modulo 2^32; f32 values are summed in float32 within a regrouping of
// the run.  The input is read once; keys_out and values_out receive only the
// runs (nothing past num_runs is written).
#include "device.hpp"
#include "launch.hpp"

namespace sca {

// Smallest tile (in vectors) of any launch shape below (11 data waves x 6
// loads x 64 lanes); scratch is sized for it.
constexpr int64_t kRbkMinTileVecs = 4224;

// The scan state of a span: run starts in it and the sum after the last one.
// V is float for f32 values and uint32_t for i32/u32 values (wrapping).
template <class V>
struct Seg {
  uint32_t c;
  V s;
  Seg() = default;
  __device__ __forceinline__ constexpr Seg(int) : c(0u), s(V(0)) {}   // the identity
  __device__ __forceinline__ constexpr Seg(uint32_t c_, V s_) : c(c_), s(s_) {}
};
static_assert(sizeof(Seg<float>) == 8 && sizeof(Seg<uint32_t>) == 8, "one 64-bit word");

// The segmented combine (a is the earlier span).  Found by argument-dependent
// lookup from the generic wave scan and look-back, and preferred over the
// generic combine as the more specialized template.
template <Op O, class V>
__device__ __forceinline__ Seg<V> combine(Seg<V> a, Seg<V> b) {
  static_assert(O == Op::Add, "reduce-by-key sums");
  const V s = b.c ? b.s : (V)(a.s + b.s);
  return Seg<V>(a.c + b.c, s);
}

template <class KF> struct KeyEq;
template <> struct KeyEq<FmtF32> {
  static __device__ __forceinline__ bool eq(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(float, a) == __builtin_bit_cast(float, b);
  }
};
template <> struct KeyEq<FmtI32> {
  static __device__ __forceinline__ bool eq(uint32_t a, uint32_t b) { return a == b; }
};
template <> struct KeyEq<FmtU32> {
  static __device__ __forceinline__ bool eq(uint32_t a, uint32_t b) { return a == b; }
};

template <class VF> struct ValT { using V = uint32_t; };
template <> struct ValT<FmtF32> { using V = float; };

template <int E>
__device__ __forceinline__ uint32_t elem(const typename VecIO<uint32_t, E>::Raw& r, int k) {
  if constexpr (E == 1) {
    return r;
  } else {
    return k == 0 ? r.x : (k == 1 ? r.y : (k == 2 ? r.z : r.w));
  }
}

// Key at window element i, or 0 bits (without touching memory) when i lies
// outside [lo, hi).  Every lane reads the same word.
__device__ __forceinline__ uint32_t key_at(uintptr_t k_base, int64_t i, int64_t lo, int64_t hi) {
  const bool in = i >= lo && i < hi;
  const Buf b(k_base + (in ? i : 0) * 4, in ? 4 : 0);
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(b.r, 0, 0, 0);
}

// FL: loads per flush of the run outputs staged in LDS; MINW: the waves per
// SIMD the register allocation must allow (two workgroups per CU).
template <class KF, class VF, int E, int WD, int K, int FL, int MINW>
__global__ __launch_bounds__(64 * (WD + 1), MINW) void reduce_by_key_kernel(
    uintptr_t k_base, uintptr_t v_base, int64_t n_cap, const int32_t* n_dev, int64_t ph,
    uintptr_t keys_out, uintptr_t values_out, uintptr_t num_runs, uint64_t* desc) {
  using V = typename ValT<VF>::V;
  using W = Seg<V>;
  using IO = VecIO<uint32_t, E>;
  using Raw = typename IO::Raw;
  constexpr int64_t VB = (int64_t)E * 4;
  constexpr int64_t kWaveVecs = (int64_t)kWave * K;
  constexpr int64_t kTileVecs = kWaveVecs * WD;
  static_assert(kTileVecs >= kRbkMinTileVecs, "scratch is sized for the smallest tile");
  __shared__ W s_wave[WD];
  __shared__ W s_prefix;
  __shared__ uint32_t s_posted;
  __shared__ uint32_t s_agg_done;
  // run outputs of FL loads per data wave (at most 64 lanes x E run starts a load)
  static_assert(K % FL == 0, "whole flushes");
  __shared__ uint32_t s_emit_k[WD][kWave * E * FL];
  __shared__ V s_emit_v[WD][kWave * E * FL];

  const int lane = lane_id(), wave = wave_id();
  const int64_t tile = blockIdx.x;
  const W id = W(0);
  const int64_t n = live_count(n_cap, n_dev);
  const int64_t lo = ph, hi = n + ph, v_last = (hi - 1) / E;
  if (n == 0 || tile * kTileVecs > v_last) {         // past the live count: nothing to do
    if (n == 0 && tile == 0 && threadIdx.x == 0) *gptr<int32_t>(num_runs) = 0;
    return;
  }
  if (threadIdx.x == 0) {
    s_posted = 0u;
    s_agg_done = 0u;
  }
  __syncthreads();

  // Run-start bits (bit k: element k of the lane's vector) of load j, whose
  // first vector is jv; `prev` is the key before the load's first element.
  auto heads = [&](int64_t jv, const Raw& rk, uint32_t prev) -> uint32_t {
    const uint32_t before = dpp<kWaveShr1, 0xf>(elem<E>(rk, E - 1), prev);
    uint32_t h = 0;
#pragma unroll
    for (int k = 0; k < E; ++k) {
      const int64_t i = (jv + lane) * E + k;
      const uint32_t p = k == 0 ? before : elem<E>(rk, k - 1);
      const bool start = (i == lo) || !KeyEq<KF>::eq(elem<E>(rk, k), p);
      h |= (i >= lo && i < hi && start) ? (1u << k) : 0u;
    }
    return h;
  };
  auto value = [&](const Raw& rv, int k, int64_t i) -> V {
    return (i >= lo && i < hi) ? __builtin_bit_cast(V, elem<E>(rv, k)) : V(0);
  };
  // Lane total of load j (elements in order).
  auto lane_total = [&](int64_t jv, const Raw& rv, uint32_t h) -> W {
    W t = id;
#pragma unroll
    for (int k = 0; k < E; ++k)
      t = combine<Op::Add>(t, W((h >> k) & 1u, value(rv, k, (jv + lane) * E + k)));
    return t;
  };

  if (wave < WD) {
    // ---- data wave ----
    // The keys of the wave's run stay in registers; the values stream in
    // after the tile's prefix is known.  A span's aggregate (c, s) needs only
    // its run starts and the values after the last of them, which almost
    // always lie in the last load: that load's values are fetched with the
    // keys.
    const int64_t wb = tile * kTileVecs + wave * kWaveVecs;
    const int64_t left = v_last + 1 - wb;
    const int64_t nv = left <= 0 ? 0 : (left < kWaveVecs ? left : kWaveVecs);
    const Buf bk(k_base + wb * VB, nv * VB), bv(v_base + wb * VB, nv * VB);
    auto vload = [&](int j) { return IO::load(bv, (uint32_t)((j * kWave + lane) * VB)); };
    Raw rk[K];
#pragma unroll
    for (int j = 0; j < K; ++j) rk[j] = IO::load(bk, (uint32_t)((j * kWave + lane) * VB));
    const Raw rv_last = vload(K - 1);
    // Wave-uniform: every element of the run is live, and the run holds
    // neither the array's first element (a run start without a key
    // comparison) nor its last (which closes the last run).  Such waves, all
    // but the first and last of the array, skip every per-element index test.
    const bool full = wb * E > lo && (wb + kWaveVecs) * E < hi;
    uint32_t prev = key_at(k_base, wb * E - 1, lo, hi);
    static_assert(K * E <= 64, "head bits of the run fit two words");
    uint64_t hb = 0u;            // bit j*E + k: element k of the lane's vector in load j starts a run
#pragma unroll
    for (int j = 0; j < K; ++j) {
      uint32_t h;
      if (full) {
        const uint32_t before = dpp<kWaveShr1, 0xf>(elem<E>(rk[j], E - 1), prev);
        h = 0u;
#pragma unroll
        for (int k = 0; k < E; ++k) {
          const uint32_t p = k == 0 ? before : elem<E>(rk[j], k - 1);
          h |= (KeyEq<KF>::eq(elem<E>(rk[j], k), p) ? 0u : 1u) << k;
        }
      } else {
        h = heads(wb + j * kWave, rk[j], prev);
      }
      hb |= (uint64_t)h << (j * E);
      prev = readlane(elem<E>(rk[j], E - 1), kWave - 1);
    }
    // the wave's aggregate: its run starts, and the sum from the last one on
    // (position (j*64 + lane)*E + k orders the wave's elements)
    const uint32_t c_w =
        readlane(wave_scan_incl<Op::Add>((uint32_t)__builtin_popcountll(hb)), kWave - 1);
    int lastpos = -1;
    if (hb != 0u) {
      const int b = 63 - __builtin_clzll(hb);
      lastpos = ((b / E) * kWave + lane) * E + b % E;
    }
    const int p_last = readlane(wave_scan_incl<Op::Max>(lastpos), kWave - 1);
    // sum of the values of load j from position p_last on (a run start's own
    // value belongs to its run; with no run start, p_last = -1 takes them all)
    auto tail_sum = [&](int j, const Raw& rv) -> V {
      V t = V(0);
#pragma unroll
      for (int k = 0; k < E; ++k) {
        const int pos = (j * kWave + lane) * E + k;
        const V v = full ? __builtin_bit_cast(V, elem<E>(rv, k))
                         : value(rv, k, (wb + j * kWave + lane) * E + k);
        t = (V)(t + (pos >= p_last ? v : V(0)));
      }
      return readlane(wave_scan_incl<Op::Add>(t), kWave - 1);
    };
    V s_w = V(0);
    constexpr int kLastStart = (K - 1) * kWave * E;
    if (p_last < kLastStart) {                 // rare: the last run started before the last load
#pragma unroll 1
      for (int j = (p_last < 0 ? 0 : p_last / (kWave * E)); j < K - 1; ++j)
        s_w = (V)(s_w + tail_sum(j, vload(j)));
    }
    s_w = (V)(s_w + tail_sum(K - 1, rv_last));
    if (lane == 0) {
      post_wave_total<Op::Add, W, WD>(W(c_w, s_w), wave, tile, s_wave, &s_posted, &s_agg_done,
                                      desc);
    }
    // the first values stream in while the look-back runs
    static_assert(K >= 3, "a ring of two values loads ahead");
    Raw ring[2];
    ring[0] = vload(0);
    ring[1] = vload(1);
    __syncthreads();
    W carry = s_prefix;
    for (int w = 0; w < wave; ++w) carry = combine<Op::Add>(carry, s_wave[w]);
    // With the exclusive state st of a run-starting element: its key opens
    // run st.c, and run st.c - 1 (if any) closed with sum st.s.  The element
    // writes both to slot st.c - base of the wave's LDS staging area, and
    // after every FL loads the wave stores the slots it filled as contiguous
    // runs of keys_out and values_out (consecutive lanes at consecutive
    // addresses) rather than one scattered store per run start.  (Run indices never
    // reach n; the bound only keeps every store inside the caller's
    // n-element outputs whatever the input.)
    uint32_t* const sk = s_emit_k[wave];
    V* const sv = s_emit_v[wave];
    uint32_t base = carry.c;                           // run index of slot 0
    auto flush = [&](uint32_t upto) {                  // upto: runs opened so far (wave-uniform)
      const uint32_t cnt = upto - base;
      // a wave's LDS operations complete in order; keep the compiler from
      // moving the reads of other lanes' slots above the writes
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      for (uint32_t i = (uint32_t)lane; i < cnt; i += kWave) {
        const uint64_t c = (uint64_t)base + i;
        if (c < (uint64_t)n) *gptr<uint32_t>(keys_out + (uintptr_t)c * 4) = sk[i];
        if (c > 0 && c - 1 < (uint64_t)n) *gptr<V>(values_out + (uintptr_t)(c - 1) * 4) = sv[i];
      }
      base = upto;
    };
    auto stage = [&](const W& st, uint32_t key) {
      const uint32_t slot = st.c - base;
      sk[slot] = key;
      sv[slot] = st.s;
    };
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const Raw rv = j == K - 1 ? rv_last : ring[j % 2];
      if (j + 2 < K - 1) ring[j % 2] = vload(j + 2);
      const int64_t jv = wb + j * kWave;
      const uint32_t h4 = (uint32_t)(hb >> (j * E)) & ((1u << E) - 1u);
      W t = id;
#pragma unroll
      for (int k = 0; k < E; ++k) {
        const V v = full ? __builtin_bit_cast(V, elem<E>(rv, k)) : value(rv, k, (jv + lane) * E + k);
        t = combine<Op::Add>(t, W((h4 >> k) & 1u, v));
      }
      const W incl = wave_scan_incl<Op::Add>(t);
      W st = combine<Op::Add>(carry, wave_shift_excl<Op::Add>(incl));
      carry = combine<Op::Add>(carry, readlane(incl, kWave - 1));
      if (full) {
#pragma unroll
        for (int k = 0; k < E; ++k) {
          const uint32_t h = (h4 >> k) & 1u;
          if (h) stage(st, elem<E>(rk[j], k));
          st = combine<Op::Add>(st, W(h, __builtin_bit_cast(V, elem<E>(rv, k))));
        }
      } else {
#pragma unroll
        for (int k = 0; k < E; ++k) {
          const int64_t i = (jv + lane) * E + k;
          const uint32_t h = (h4 >> k) & 1u;
          if (h) stage(st, elem<E>(rk[j], k));
          st = combine<Op::Add>(st, W(h, value(rv, k, i)));
          // the last element closes the last run
          if (i == hi - 1 && st.c >= 1 && st.c <= (uint64_t)n) {
            *gptr<V>(values_out + (uintptr_t)(st.c - 1) * 4) = st.s;
            *gptr<int32_t>(num_runs) = (int32_t)st.c;
          }
        }
      }
      if ((j + 1) % FL == 0 && carry.c != base) flush(carry.c);
    }
  } else {
    // ---- look-back wave ----
    auto tile_agg = [&]() {
      W a = s_wave[0];
#pragma unroll
      for (int w = 1; w < WD; ++w) a = combine<Op::Add>(a, s_wave[w]);
      return a;
    };
    W prefix = id;
    if (tile > 0) {
      // fallback for a late predecessor: fold its input in element order, a
      // few loads at a time (this rare path must not raise the kernel's
      // register count, which sets how many workgroups fit on a CU).  Counts
      // and integer sums are exactly what that tile would publish; float32
      // sums are grouped differently from its data waves' tail sums, so they
      // may differ in the last bits (within the float-add tolerance)
      auto reduce_tile = [&](int64_t t) -> W {
        constexpr int kG = 2;
        static_assert(kTileVecs % (kG * kWave) == 0, "whole groups of loads");
        const int64_t first = t * kTileVecs;
        const int64_t left = v_last + 1 - first;
        const int64_t nv = left <= 0 ? 0 : (left < kTileVecs ? left : kTileVecs);
        const Buf bk(k_base + first * VB, nv * VB), bv(v_base + first * VB, nv * VB);
        W acc = id;
        uint32_t prev = key_at(k_base, first * E - 1, lo, hi);
#pragma unroll 1
        for (int g = 0; g < (int)(kTileVecs / (kG * kWave)); ++g) {
          Raw rk[kG], rv[kG];
#pragma unroll
          for (int j = 0; j < kG; ++j) {
            const uint32_t off = (uint32_t)(((g * kG + j) * kWave + lane) * VB);
            rk[j] = IO::load(bk, off);
            rv[j] = IO::load(bv, off);
          }
#pragma unroll
          for (int j = 0; j < kG; ++j) {
            const int64_t jv = first + (g * kG + j) * kWave;
            const uint32_t h = heads(jv, rk[j], prev);
            prev = readlane(elem<E>(rk[j], E - 1), kWave - 1);
            acc = combine<Op::Add>(
                acc, readlane(wave_scan_incl<Op::Add>(lane_total(jv, rv[j], h)), kWave - 1));
          }
        }
        return acc;
      };
      prefix = look_back<Op::Add, W, kPollShort>(desc, tile, kLookBackTimeout, reduce_tile);
    }
    while (!lds_flag_set(&s_agg_done)) __builtin_amdgcn_s_sleep(1);
    if (lane == 0) {
      Desc<W>::publish(desc, tile, kInc, combine<Op::Add>(prefix, tile_agg()));
      s_prefix = prefix;
    }
    __syncthreads();
  }
}

__global__ void rbk_count_zero_kernel(int32_t* num_runs) { *num_runs = 0; }

// Tiles of tv vectors covering window elements [ph, n + ph) in vectors of e.
static int64_t rbk_tiles_for(int64_t n, int64_t ph, int e, int64_t tv) {
  if (n <= 0) return 0;
  const int64_t v_last = (n + ph - 1) / e;
  return v_last / tv + 1;
}

// Sized for the one-element-per-vector path (no phase) and the smallest tile;
// four-element vectors at a phase below 32 elements never need more tiles.
size_t reduce_by_key_tiles(int64_t n) { return (size_t)rbk_tiles_for(n, 0, 1, kRbkMinTileVecs); }

template <class KF, class VF, int WD, int K, int FL, int MINW>
static hipError_t launch_rbk_cfg(const void* keys, const void* values, void* keys_out,
                                 void* values_out, int32_t* num_runs, int64_t n, void* scratch,
                                 hipStream_t stream, const int32_t* n_dev) {
  constexpr int64_t TV = (int64_t)kWave * WD * K;
  const uintptr_t ka = (uintptr_t)keys, va = (uintptr_t)values;
  const bool vec = (ka % 16) == (va % 16);
  const int e = vec ? 4 : 1;
  // the window starts on the 128-byte line of the first key when the values
  // share its place in a line (the elements before the arrays are read within
  // their first lines, so within their pages, and take no part in any run)
  const bool line = (ka % 128) == (va % 128);
  const int64_t ph = vec ? (int64_t)((ka % (line ? 128 : 16)) / 4) : 0;
  const int64_t ntiles = rbk_tiles_for(n, ph, e, TV);
  uint64_t* desc = desc_base(scratch);
  hipError_t err = launch_fill_desc(desc, ntiles, Desc<Seg<float>>::kWords, stream);
  if (err != hipSuccess) return err;
  const dim3 grid((unsigned)ntiles), block(64 * (WD + 1));
  const uintptr_t ko = (uintptr_t)keys_out, vo = (uintptr_t)values_out, nr = (uintptr_t)num_runs;
  if (vec) {
    reduce_by_key_kernel<KF, VF, 4, WD, K, FL, MINW><<<grid, block, 0, stream>>>(
        ka - ph * 4, va - ph * 4, n, n_dev, ph, ko, vo, nr, desc);
  } else {
    reduce_by_key_kernel<KF, VF, 1, WD, K, FL, MINW><<<grid, block, 0, stream>>>(
        ka, va, n, n_dev, 0, ko, vo, nr, desc);
  }
  return hipGetLastError();
}

template <class KF, class VF>
static hipError_t launch_rbk_t(const void* keys, const void* values, void* keys_out,
                               void* values_out, int32_t* num_runs, int64_t n, void* scratch,
                               hipStream_t stream, const int32_t* n_dev) {
  // Launch shape measured on MI355X over 2^27 pairs in runs of mean length 8
  // (us, u32 values): 11 data waves x 6 loads with two workgroups per CU and
  // the run outputs flushed every 3 loads 252-255; every 1 / 2 loads 273-277 /
  // 263; once per wave (132 KiB of LDS, one workgroup per CU) 320.  7 x 8 (2
  // loads per flush) 263, 15 x 8 (one workgroup per CU) 276-281, 11 x 4
  // 277, 13 x 6 283 (20 bytes spilled).  The earlier kernel, with one
  // scattered store per run start: 15 x 8 285-294, 11 x 8 at two per CU 277-281.
  return launch_rbk_cfg<KF, VF, 11, 6, 3, 6>(keys, values, keys_out, values_out, num_runs, n,
                                             scratch, stream, n_dev);
}

template <class KF>
static hipError_t launch_rbk_k(const void* keys, const void* values, void* keys_out,
                               void* values_out, int32_t* num_runs, int64_t n, Fmt vfmt,
                               void* scratch, hipStream_t stream, const int32_t* n_dev) {
  switch (vfmt) {
    case Fmt::F32:
      return launch_rbk_t<KF, FmtF32>(keys, values, keys_out, values_out, num_runs, n, scratch,
                                      stream, n_dev);
    default:   // i32 and u32 values share the wrapping add
      return launch_rbk_t<KF, FmtU32>(keys, values, keys_out, values_out, num_runs, n, scratch,
                                      stream, n_dev);
  }
}

hipError_t launch_reduce_by_key(const void* keys, const void* values, void* keys_out,
                                void* values_out, int32_t* num_runs, int64_t n, Fmt kfmt,
                                Fmt vfmt, void* scratch, hipStream_t stream,
                                const int32_t* n_dev) {
  if (n == 0) {
    rbk_count_zero_kernel<<<dim3(1), dim3(1), 0, stream>>>(num_runs);
    return hipGetLastError();
  }
  switch (kfmt) {
    case Fmt::F32:
      return launch_rbk_k<FmtF32>(keys, values, keys_out, values_out, num_runs, n, vfmt, scratch,
                                  stream, n_dev);
    default:   // i32 and u32 keys compare as bits
      return launch_rbk_k<FmtU32>(keys, values, keys_out, values_out, num_runs, n, vfmt, scratch,
                                  stream, n_dev);
  }
}

}  // namespace sca
