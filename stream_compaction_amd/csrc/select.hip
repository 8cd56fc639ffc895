// Stream compaction ("Algorithms" page, Quadrants user guide, section
// qd.algorithms.select): the flagged elements, in input order, become the
// dense prefix out[0..k) and k goes to num_out[0].
//
// The page's own realization is three phases (exclusive scan of the flags
// into an n-entry index buffer, scatter, one-thread count; section "Under the
// hood").  Here one kernel does all of it in a single pass, with the scan of
// the flag counts done by DPP wave scans and the same decoupled look-back as
// the device-wide scan, and no index buffer.
//
// A tile's count depends on its flag bytes alone, so the tile is ordered
// around them.  Workgroup b owns tile b: WD data waves and one look-back wave.
// Each data wave owns a run of C chunks; a chunk is J payload vectors per lane
// (load j of lane l is vector j*64 + l of the chunk, so one load instruction
// covers 64 consecutive vectors).  A vector is 16 bytes for elements of 4, 8
// and 16 bytes, and four elements (4 or 8 bytes) for elements of 1 and 2.
//   1. A data wave loads the flags of its whole run (E bytes per payload
//      vector), forms the selection masks, and posts its count; the last data
//      wave to post publishes the tile's count, one flag round trip after the
//      tile starts.  It then issues the payload loads of its first chunks.
//      A lane loads a payload vector only when one of its elements is
//      selected: the other lanes point the load past the buffer's end, where
//      it reads zero without touching memory, so at low selectivity most of
//      the payload is never fetched.
//   2. The look-back wave walks back over the predecessors' descriptors from
//      the start, publishes the tile's inclusive count and hands over the
//      tile's output offset; the tile with the last id writes num_out.
//   3. Each data wave then streams its chunks, keeping the payload of the next
//      two chunks in flight: ranks within the chunk come from DPP scans of the
//      lane counts; the selected elements are packed into the wave's own LDS
//      staging area at their rank, shifted so LDS vectors line up with the
//      vectors of `out`, and the wave stores the whole 128-byte lines the
//      chunk completed with whole-vector stores; the unfinished line is
//      carried in LDS into the next chunk, so a wave writes partial vectors
//      and lines (element by element) only at the two ends of its output.
//      Unselected elements are written to a per-lane discard slot, and stores
//      without data point past the buffer's end, so every chunk issues the
//      same instructions whatever the flags hold.
// Elements move as raw bits, so any type of 1, 2, 4, 8 or 16 bytes (NaN
// payloads and structs included) is copied exactly.  out past the count is
// never written.
#include "device.hpp"
#include "launch.hpp"

namespace sca {

template <int EB> struct Bits;
template <> struct Bits<1> { using T = uint8_t; };
template <> struct Bits<2> { using T = uint16_t; };
template <> struct Bits<4> { using T = uint32_t; };
template <> struct Bits<8> { using T = uint64_t; };
template <> struct Bits<16> { using T = u32x4; };

// Elements per payload vector: four for elements of 1, 2 and 4 bytes (vectors
// of 4, 8 and 16 bytes), two for 8-byte and one for 16-byte elements.  A
// vector's flags are then at most 4 bytes, and a lane's count per load at
// most 4, which the byte-packed rank scan below relies on.
template <int EB> constexpr int sel_e() { return EB <= 4 ? 4 : 16 / EB; }

// A payload vector of VB bytes as loaded and stored (4, 8 or 16 bytes).
template <int VB> struct SelVec;
template <> struct SelVec<4> { using T = uint32_t; };
template <> struct SelVec<8> { using T = u32x2; };
template <> struct SelVec<16> { using T = u32x4; };

template <int VB>
__device__ __forceinline__ typename SelVec<VB>::T sel_load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (VB == 4) {
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kNT);
  } else if constexpr (VB == 8) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kNT));
  } else {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kNT));
  }
}

// One element (B bytes) or one vector stored at byte offset off.
template <int B, class V>
__device__ __forceinline__ void sel_store(V v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (B == 1) {
    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)v, r, off, 0, kStoreAux);
  } else if constexpr (B == 2) {
    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)v, r, off, 0, kStoreAux);
  } else if constexpr (B == 4) {
    __builtin_amdgcn_raw_buffer_store_b32((uint32_t)v, r, off, 0, kStoreAux);
  } else if constexpr (B == 8) {
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, off, 0, kStoreAux);
  } else {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, kStoreAux);
  }
}

constexpr int kSelJ = 4;   // payload vectors per lane per chunk

// Scratch is sized for tiles of at least this many 16-byte payload vectors
// (the launch shape below: 8 data waves x 8 chunks x 4 loads x 64 lanes).
constexpr int64_t kSelMinTileVecs = 16384;

// A buffer offset far past any buffer's range: loads there read zero and
// stores are dropped, without a memory access.  It stays below 2^32 after the
// compiler adds an immediate offset (at most 4095), so it cannot wrap into
// the range.
constexpr uint32_t kOffNone = 0x80000000u;

template <int EB, bool FVEC, int WD, int C>
__global__ __launch_bounds__(64 * (WD + 1)) void select_kernel(uintptr_t in_base, uintptr_t flags_base,
                                                         uintptr_t out_base, int64_t n_cap,
                                                         const int32_t* n_dev, int64_t ph,
                                                         int64_t out_ph, int32_t* num_out,
                                                         uint64_t* desc) {
  using T = typename Bits<EB>::T;
  constexpr int E = sel_e<EB>();                  // elements per payload vector
  constexpr int VB = E * EB;                      // bytes per payload vector
  using V = typename SelVec<VB>::T;
  constexpr int J = kSelJ;
  constexpr int64_t kChunkVecs = (int64_t)kWave * J;
  constexpr int64_t kWaveVecs = kChunkVecs * C;
  constexpr int64_t kTileVecs = kWaveVecs * WD;
  static_assert(kTileVecs >= kSelMinTileVecs, "scratch is sized for the smallest tile");
  // staging slots per wave: one chunk of elements plus the unfinished line
  // carried from the previous chunk (or the slots before the wave's first
  // output position in its first line), fewer than 128 bytes
  constexpr int kStage = (int)kChunkVecs * E + 128 / EB;
  constexpr int kStageVecs = kStage / E;
  constexpr int kStoreIters = (kStageVecs + kWave - 1) / kWave;
  __shared__ __attribute__((aligned(16))) T s_stage[WD][kStage];
  __shared__ T s_discard[WD][kWave];
  __shared__ uint32_t s_wave[WD];
  __shared__ uint32_t s_prefix;
  __shared__ uint32_t s_posted;   // data waves whose counts are in s_wave
  __shared__ uint32_t s_agg_done; // the tile's count is published

  const int lane = lane_id(), wave = wave_id();
  const int64_t tile = blockIdx.x;
  const int64_t n = live_count(n_cap, n_dev);
  const int64_t lo = ph, hi = n + ph, v_last = (hi - 1) / E;
  const int64_t ntiles = n == 0 ? 0 : v_last / kTileVecs + 1;   // tiles holding live elements
  if (tile >= ntiles) {                              // past the live count: nothing to do
    if (n == 0 && tile == 0 && threadIdx.x == 0) *num_out = 0;
    return;
  }
  if (threadIdx.x == 0) {
    s_posted = 0u;
    s_agg_done = 0u;
  }
  __syncthreads();

  // Flag bytes of payload vector u of buffer fb, whose first element is
  // window element e0 (E bytes, low byte first; zero past the buffer's range).
  // Aligned flags load whole naturally aligned words; otherwise bytes are
  // loaded one by one, and only those of live elements, so no byte outside
  // the flags array is read.
  auto flag_word = [&](const Buf& fb, uint32_t u, int64_t e0) -> uint32_t {
    if constexpr (FVEC && E == 4) {
      (void)e0;
      return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(fb.r, u * 4, 0, kNT);
    } else if constexpr (FVEC && E == 2) {
      (void)e0;
      return (uint32_t)(uint16_t)__builtin_amdgcn_raw_buffer_load_b16(fb.r, u * 2, 0, kNT);
    } else if constexpr (E == 1) {
      (void)e0;     // one flag per vector: every loaded vector's element is live
      return (uint32_t)(uint8_t)__builtin_amdgcn_raw_buffer_load_b8(fb.r, u, 0, kNT);
    } else {
      uint32_t f = 0u;
#pragma unroll
      for (int k = 0; k < E; ++k) {
        const bool live = e0 + k >= lo && e0 + k < hi;
        f |= (uint32_t)(uint8_t)__builtin_amdgcn_raw_buffer_load_b8(
                 fb.r, live ? u * E + k : kOffNone, 0, kNT)
             << (8 * k);
      }
      return f;
    }
  };
  // Selection bits of one payload vector from its flag word f: bit 8k + 7 is
  // set when flag byte k is nonzero (per byte, (b & 0x7f) + 0x7f sets bit 7
  // for any nonzero low bits and never carries into the next byte).  With
  // jv the first vector of its load (wave-uniform) and `full` telling that
  // every element of the wave's run is live, elements outside [lo, hi) are
  // cleared only on the slow path.
  constexpr uint32_t kTop = E == 4 ? 0x80808080u : (E == 2 ? 0x8080u : 0x80u);   // bit 7 of each flag byte
  auto sel_bits = [&](int64_t jv, uint32_t f, bool full) {
    uint32_t t = (((f & 0x7f7f7f7fu) + 0x7f7f7f7fu) | f) & kTop;
    if (!full && !(jv * E >= lo && (jv + kWave) * E <= hi)) {   // wave-uniform
      const int64_t e0 = (jv + lane) * E;
      uint32_t live = 0u;
#pragma unroll
      for (int k = 0; k < E; ++k) live |= (e0 + k >= lo && e0 + k < hi ? 1u : 0u) << (8 * k + 7);
      t &= live;
    }
    return t;
  };
  // The buffer over `len` vectors of the run starting at vector `first`
  // (clamped to the live vectors), for an array of `vb`-byte vectors at `base`.
  auto run_buf = [&](uintptr_t base, int64_t vb, int64_t first, int64_t len) {
    const int64_t left = v_last + 1 - first;
    const int64_t nv = left <= 0 ? 0 : (left < len ? left : len);
    return Buf(base + first * vb, nv * vb);
  };

  const int64_t wb = tile * kTileVecs + wave * kWaveVecs;  // this data wave's first vector
  // sb[c]: selection bits of chunk c; element k of the lane's vector j is
  // selected when bit 8k + 7 - j is set
  uint32_t sb[C];
  V pay[C][J];             // payload (only the chunks in flight are live)
  const Buf pbuf = run_buf(in_base, VB, wb, kWaveVecs);
  auto load_chunk = [&](int c) {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const uint32_t off = (uint32_t)(((c * J + j) * kWave + lane) * VB);
      const bool any = (sb[c] & (kTop >> j)) != 0u;
      pay[c][j] = sel_load<VB>(pbuf.r, any ? off : kOffNone);
    }
  };

  if (wave < WD) {
    // 1. flags of the whole run -> selection bits -> the wave's count
    const Buf fbuf = run_buf(flags_base, E, wb, kWaveVecs);
    const bool full = wb * E >= lo && (wb + kWaveVecs) * E <= hi;   // every element live
    uint32_t f[C][J];
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int u = (c * J + j) * kWave + lane;
        f[c][j] = flag_word(fbuf, (uint32_t)u, (wb + u) * E);
      }
    uint32_t cnt = 0u;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      sb[c] = 0u;
#pragma unroll
      for (int j = 0; j < J; ++j) sb[c] |= sel_bits(wb + (c * J + j) * kWave, f[c][j], full) >> j;
      cnt += (uint32_t)__builtin_popcount(sb[c]);
    }
    const uint32_t total = readlane(wave_scan_incl<Op::Add>(cnt), kWave - 1);
    if (lane == 0) {
      post_wave_total<Op::Add, uint32_t, WD>(total, wave, tile, s_wave, &s_posted, &s_agg_done,
                                             desc);
    }
    load_chunk(0);
    if constexpr (C > 1) load_chunk(1);
  } else {
    // 2. the look-back wave: walks back from the start and, once the last
    //    data wave has published the tile's count, publishes the tile's
    //    inclusive count and hands over the output offset
    uint32_t prefix = 0u;
    if (tile > 0) {
      // fallback for a late predecessor: count its selected flags, one chunk
      // (J loads) at a time
      auto reduce_tile = [&](int64_t t) -> uint32_t {
        uint32_t acc = 0u;
#pragma unroll 1
        for (int g = 0; g < WD * C; ++g) {
          const int64_t first = t * kTileVecs + (int64_t)g * kChunkVecs;
          const Buf fb = run_buf(flags_base, E, first, kChunkVecs);
          uint32_t c = 0u;
#pragma unroll
          for (int j = 0; j < J; ++j)
            c += (uint32_t)__builtin_popcount(sel_bits(
                first + j * kWave,
                flag_word(fb, (uint32_t)(j * kWave + lane), (first + j * kWave + lane) * E),
                false));
          acc += readlane(wave_scan_incl<Op::Add>(c), kWave - 1);
        }
        return acc;
      };
      prefix = look_back<Op::Add, uint32_t, kPollLong>(desc, tile, kLookBackTimeout, reduce_tile);
    }
    while (!lds_flag_set(&s_agg_done)) __builtin_amdgcn_s_sleep(1);
    if (lane == 0) {
      uint32_t agg = 0u;
#pragma unroll
      for (int w = 0; w < WD; ++w) agg += s_wave[w];
      Desc<uint32_t>::publish(desc, tile, kInc, prefix + agg);
      s_prefix = prefix;
      if (tile == ntiles - 1) *num_out = (int32_t)(prefix + agg);
    }
  }
  __syncthreads();
  if (wave >= WD) return;

  // 3. stream the chunks: rank, pack into LDS, store the run.  The wave's
  // LDS staging area starts at a 128-byte line of `out` (slot 0 is the
  // element at window position `base`), and every chunk stores only the
  // whole lines it has completed; the partial line at the end moves to the
  // front of the staging area and is completed by the next chunk.  So the
  // wave writes whole lines except at the two ends of its output range.
  constexpr int LE = 128 / EB;                        // elements per 128-byte line
  static_assert(LE % E == 0, "a line is whole vectors");
  uint32_t r0 = s_prefix;                             // output index of the wave's first selected element
  for (int w = 0; w < wave; ++w) r0 += s_wave[w];
  r0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)r0);   // wave-uniform: buffer bases use it
  T* const stage = s_stage[wave];
  // window position P lies at a line start when (out_base + P * EB) % 128 == 0
  const int lphase = (int)((out_base % 128) / EB);
  const int64_t p_valid = (int64_t)r0 + out_ph;       // the wave's first output position
  int64_t base = p_valid - (p_valid + lphase) % LE;   // line-aligned position of slot 0
  int fill = (int)(p_valid - base);                   // slot of the next kept element
#pragma unroll
  for (int c = 0; c < C; ++c) {
    if (c + 2 < C) load_chunk(c + 2);
    const int s = fill;
    // ranks: the chunk's elements are ordered load by load, then lane by
    // lane.  The lane's J counts (at most E each) are packed in bytes and
    // scanned exclusively in one pass: a byte then sums at most 63 lanes'
    // counts (at most 252), so bytes never carry into each other.
    uint32_t cpk = 0u;
#pragma unroll
    for (int j = 0; j < J; ++j)
      cpk |= (uint32_t)__builtin_popcount(sb[c] & (kTop >> j)) << (8 * j);
    const uint32_t ex = wave_scan_incl<Op::Add>(dpp<kWaveShr1, 0xf>(cpk, 0u));
    const uint32_t e63 = readlane(ex, kWave - 1), c63 = readlane(cpk, kWave - 1);
    uint32_t pos[J];
    uint32_t run = (uint32_t)s;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      pos[j] = run + ((ex >> (8 * j)) & 0xffu);
      run += ((e63 >> (8 * j)) & 0xffu) + ((c63 >> (8 * j)) & 0xffu);
    }
    const int end = (int)run;                 // one past the last staged slot
    // pack: selected elements to their slots, the others to the discard slot
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const V r = pay[c][j];
      T x[E];
      if constexpr (EB == 1) {
#pragma unroll
        for (int k = 0; k < 4; ++k) x[k] = (uint8_t)(r >> (8 * k));
      } else if constexpr (EB == 2) {
        x[0] = (uint16_t)r.x; x[1] = (uint16_t)(r.x >> 16);
        x[2] = (uint16_t)r.y; x[3] = (uint16_t)(r.y >> 16);
      } else if constexpr (EB == 4) {
        x[0] = r.x; x[1] = r.y; x[2] = r.z; x[3] = r.w;
      } else if constexpr (EB == 8) {
        x[0] = ((uint64_t)r.y << 32) | r.x;
        x[1] = ((uint64_t)r.w << 32) | r.z;
      } else {
        x[0] = r;
      }
      uint32_t p = pos[j];
#pragma unroll
      for (int k = 0; k < E; ++k) {
        const bool sel = (sb[c] >> (8 * k + 7 - j)) & 1u;
        *(sel ? &stage[p] : &s_discard[wave][lane]) = x[k];
        p += sel ? 1u : 0u;
      }
    }
    // a wave's LDS operations complete in order; wait for the writes before
    // the reads of other lanes' slots
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    // store slots [first, cut): whole lines, or everything at the wave's last
    // chunk; slots below the wave's first output position are not its own
    const int cut = c == C - 1 ? end : end / LE * LE;
    const int first = (int)(p_valid > base ? p_valid - base : 0);
    const int nvec = (cut + E - 1) / E;
    const Buf ob(out_base + (base / E) * VB, (int64_t)nvec * VB);
#pragma unroll
    for (int i = 0; i < kStoreIters; ++i) {
      const int q = lane + i * kWave;
      const bool full = q * E >= first && (q + 1) * E <= cut;
      const int qr = q < kStageVecs ? q : kStageVecs - 1;
      const V v = *(const V*)&stage[qr * E];
      sel_store<VB>(v, ob.r, full ? (uint32_t)(q * VB) : kOffNone);
    }
    // the partial vectors: the first (lane 0) and the last (lane 1), element by element
    {
      const int q = lane == 0 ? first / E : nvec - 1;
      const bool partial = (lane == 0 || (lane == 1 && nvec - 1 != first / E)) && cut > first &&
                           !(q * E >= first && (q + 1) * E <= cut);
#pragma unroll
      for (int k = 0; k < E; ++k) {
        const int slot = q * E + k;
        const bool ok = partial && slot >= first && slot < cut;
        const T v = stage[ok ? slot : 0];
        const uint32_t off = ok ? (uint32_t)(slot * EB) : kOffNone;
        sel_store<EB>(v, ob.r, off);
      }
    }
    // the unfinished line moves to the front (fewer than LE slots, read from
    // slot cut >= LE on, so source and destination never overlap)
    if (c < C - 1 && cut > 0) {
      const int cnt = end - cut;
      constexpr int kMoveIters = (LE + kWave - 1) / kWave;
      T t[kMoveIters];
#pragma unroll
      for (int i = 0; i < kMoveIters; ++i) {
        const int q = lane + i * kWave;
        t[i] = stage[q < cnt ? cut + q : 0];
      }
#pragma unroll
      for (int i = 0; i < kMoveIters; ++i) {
        const int q = lane + i * kWave;
        if (q < cnt) stage[q] = t[i];
      }
      base += cut;
      fill = cnt;
    } else {
      fill = end;
    }
  }
}

// Tiles of tv vectors covering window elements [ph, n + ph) in vectors of e.
static int64_t sel_tiles_for(int64_t n, int64_t ph, int e, int64_t tv) {
  if (n <= 0) return 0;
  const int64_t v_last = (n + ph - 1) / e;
  return v_last / tv + 1;
}

// Sized for 16-byte elements (one per vector, the most tiles) at the largest
// window phase they can take (seven vectors into a line) and the smallest
// tile, so one scratch size serves every element width, alignment and launch
// shape.
size_t select_tiles(int64_t n, size_t elem_bytes) {
  (void)elem_bytes;
  return (size_t)sel_tiles_for(n, 7, 1, kSelMinTileVecs);
}

__global__ void store_count_zero_kernel(int32_t* num_out) { *num_out = 0; }

// One launch shape: WD data waves (plus the look-back wave), C chunks per
// data wave.
template <int EB, int WD, int C>
static hipError_t launch_sel_cfg(const void* in, const uint8_t* flags, void* out, int32_t* num_out,
                                 int64_t n, void* scratch, hipStream_t stream,
                                 const int32_t* n_dev) {
  constexpr int E = sel_e<EB>(), VB = E * EB;
  constexpr int64_t TV = (int64_t)kWave * kSelJ * C * WD;
  const uintptr_t ia = (uintptr_t)in, fa = (uintptr_t)flags, oa = (uintptr_t)out;
  // The payload window starts on the payload vector that holds the first
  // element or, when the flags before the array's first flag stay inside the
  // flags' own 128-byte line (so inside their page), on the payload's 128-byte
  // line, so that every payload load covers whole lines.  The elements before
  // the array are never selected.
  const int64_t lph = (int64_t)((ia % 128) / EB);
  const int64_t ph = (int64_t)(fa % 128) >= lph ? lph : (int64_t)((ia % VB) / EB);
  const int64_t out_ph = (int64_t)((oa % VB) / EB);
  const uintptr_t fbase = fa - (uintptr_t)ph;          // flag byte of window element 0
  const bool fvec = (fbase % E) == 0;
  const int64_t ntiles = sel_tiles_for(n, ph, E, TV);
  uint64_t* desc = desc_base(scratch);
  hipError_t err = launch_fill_desc(desc, ntiles, Desc<uint32_t>::kWords, stream);
  if (err != hipSuccess) return err;
  const dim3 grid((unsigned)ntiles), block(64 * (WD + 1));
  const uintptr_t ibase = ia - (uintptr_t)ph * EB, obase = oa - (uintptr_t)out_ph * EB;
  if (fvec) {
    select_kernel<EB, true, WD, C><<<grid, block, 0, stream>>>(ibase, fbase, obase, n, n_dev, ph,
                                                              out_ph, num_out, desc);
  } else {
    select_kernel<EB, false, WD, C><<<grid, block, 0, stream>>>(ibase, fbase, obase, n, n_dev, ph,
                                                               out_ph, num_out, desc);
  }
  return hipGetLastError();
}

template <int EB>
static hipError_t launch_sel_t(const void* in, const uint8_t* flags, void* out, int32_t* num_out,
                               int64_t n, void* scratch, hipStream_t stream,
                               const int32_t* n_dev) {
  return launch_sel_cfg<EB, 8, 8>(in, flags, out, num_out, n, scratch, stream, n_dev);
}

hipError_t launch_select(const void* in, const uint8_t* flags, void* out, int32_t* num_out,
                         int64_t n, size_t elem_bytes, void* scratch, hipStream_t stream,
                         const int32_t* n_dev) {
  if (n == 0) {
    store_count_zero_kernel<<<dim3(1), dim3(1), 0, stream>>>(num_out);
    return hipGetLastError();
  }
  switch (elem_bytes) {
    case 1: return launch_sel_t<1>(in, flags, out, num_out, n, scratch, stream, n_dev);
    case 2: return launch_sel_t<2>(in, flags, out, num_out, n, scratch, stream, n_dev);
    case 4: return launch_sel_t<4>(in, flags, out, num_out, n, scratch, stream, n_dev);
    case 8: return launch_sel_t<8>(in, flags, out, num_out, n, scratch, stream, n_dev);
    default: return launch_sel_t<16>(in, flags, out, num_out, n, scratch, stream, n_dev);
  }
}

}  // namespace sca
