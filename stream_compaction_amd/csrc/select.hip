// Stream compaction ("Algorithms" page, Quadrants user guide, section
// qd.algorithms.select): the flagged elements, in input order, become the
// dense prefix out[0..k) and k goes to num_out[0].
//
// The page's own realization is three phases (exclusive scan of the flags
// into an n-entry index buffer, scatter, one-thread count; section "Under the
// hood").  Here one kernel does all of it in a single pass, with the scan of
// the flag counts done by the same DPP wave scan and decoupled look-back as
// the device-wide scan, and no index buffer.  Workgroup b owns tile b; it has
// WD data waves and one look-back wave:
//   1. each data wave loads 16-byte payload vectors (load j of lane l is
//      vector j*64 + l of its run) and the matching flag bytes, and forms a
//      bit mask of its selected elements;
//   2. lane counts are scanned across the wave (DPP) and posted to LDS; the
//      last data wave to post publishes the tile's count; the look-back wave,
//      walking back over the predecessors' descriptors from the start, then
//      publishes the tile's inclusive count and hands over the tile's output
//      offset G; the tile with the last id writes num_out;
//   3. selected elements are packed into LDS at their rank, shifted so LDS
//      vectors line up with 16-byte vectors of `out`, and the workgroup
//      stores the packed run [G, G + count) with 16-byte stores (element
//      stores only for the partial vectors at its two ends).
// Elements move as raw bits, so any 4- or 8-byte type (NaN payloads
// included) is copied exactly.  out past the count is never written.
#include "device.hpp"
#include "launch.hpp"

namespace sca {

// Smallest tile (in vectors) of any launch shape below (3 data waves x 12
// loads x 64 lanes); scratch is sized for it.
constexpr int64_t kSelMinTileVecs = 2304;

template <int EB> struct Bits;
template <> struct Bits<4> { using T = uint32_t; };
template <> struct Bits<8> { using T = uint64_t; };

template <int EB, int E, bool FVEC, int WD, int K>
__global__ __launch_bounds__(64 * (WD + 1)) void select_kernel(uintptr_t in_base, uintptr_t flags_base,
                                                         uintptr_t out_base, int64_t n_cap,
                                                         const int32_t* n_dev, int64_t ph,
                                                         int64_t out_ph, int32_t* num_out,
                                                         uint64_t* desc) {
  using T = typename Bits<EB>::T;
  constexpr int EO = 16 / EB;                     // elements per 16-byte output vector
  constexpr int kThreads = kWave * (WD + 1);
  constexpr int64_t kWaveVecs = (int64_t)kWave * K;
  constexpr int64_t kTileVecs = kWaveVecs * WD;
  static_assert(kTileVecs >= kSelMinTileVecs, "scratch is sized for the smallest tile");
  constexpr int kTileElems = (int)kTileVecs * E;
  constexpr int64_t VB = (int64_t)E * EB;
  __shared__ __attribute__((aligned(16))) T s_stage[kTileElems + EO];
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

  // Flag bytes of the run of 64*K vectors starting at `first` (E bytes per
  // vector, packed low byte first; zero past v_last).
  auto load_flags = [&](int64_t first, uint32_t (&f)[K]) {
    const int64_t left = v_last + 1 - first;
    const int64_t nv = left <= 0 ? 0 : (left < kWaveVecs ? left : kWaveVecs);
    const Buf fbuf(flags_base + first * E, nv * E);
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const uint32_t u = (uint32_t)(j * kWave + lane);
      if constexpr (FVEC && E == 4) {
        f[j] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(fbuf.r, u * 4, 0, kNT);
      } else if constexpr (FVEC && E == 2) {
        f[j] = (uint32_t)(uint16_t)__builtin_amdgcn_raw_buffer_load_b16(fbuf.r, u * 2, 0, kNT);
      } else {
        f[j] = 0u;
#pragma unroll
        for (int k = 0; k < E; ++k)
          f[j] |= (uint32_t)(uint8_t)__builtin_amdgcn_raw_buffer_load_b8(fbuf.r, u * E + k, 0, kNT)
                  << (8 * k);
      }
    }
  };
  // Selection mask (bit k = element k) of the lane's vector in load j.
  auto select_mask = [&](int64_t jv, uint32_t f) {
    uint32_t m = 0u;
#pragma unroll
    for (int k = 0; k < E; ++k) m |= (((f >> (8 * k)) & 0xffu) != 0u ? 1u : 0u) << k;
    if (!(jv * E >= lo && (jv + kWave) * E <= hi)) {   // wave-uniform: some vector is partial
      const int64_t e0 = (jv + lane) * E;
      const int64_t ks = lo - e0, ke = hi - e0;
      const uint32_t start = ks <= 0 ? 0u : (ks >= E ? (uint32_t)E : (uint32_t)ks);
      const uint32_t end = ke <= 0 ? 0u : (ke >= E ? (uint32_t)E : (uint32_t)ke);
      m &= ((1u << end) - 1u) & ~((1u << start) - 1u);
    }
    return m;
  };

  // 1. payload and selection masks (data waves): every load is issued
  //    unconditionally through buffer resources that end at the wave's last
  //    valid vector (past it: zero bits, i.e. unselected); only the two end
  //    vectors of the array need masking
  const int64_t wb = tile * kTileVecs + wave * kWaveVecs;  // this wave's first vector
  T x[K][E];
  uint32_t m[K];
  uint32_t pre[K];
  if (wave < WD) {
    uint32_t f[K];
    {
      const int64_t left = v_last + 1 - wb;
      const int64_t nv = left <= 0 ? 0 : (left < kWaveVecs ? left : kWaveVecs);
      const Buf pbuf(in_base + wb * VB, nv * VB);
#pragma unroll
      for (int j = 0; j < K; ++j) {
        const uint32_t u = (uint32_t)(j * kWave + lane);
        if constexpr (E == 1) {
          if constexpr (EB == 4) {
            x[j][0] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(pbuf.r, u * 4, 0, kNT);
          } else {
            x[j][0] = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(pbuf.r, u * 8, 0, kNT));
          }
        } else {
          const uint4 r = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(pbuf.r, u * 16, 0, kNT));
          if constexpr (EB == 4) {
            x[j][0] = r.x; x[j][1] = r.y; x[j][2] = r.z; x[j][3] = r.w;
          } else {
            x[j][0] = ((uint64_t)r.y << 32) | r.x;
            x[j][1] = ((uint64_t)r.w << 32) | r.z;
          }
        }
      }
    }
    load_flags(wb, f);
#pragma unroll
    for (int j = 0; j < K; ++j) m[j] = select_mask(wb + j * kWave, f[j]);

    // 2. ranks within the wave; the wave's count goes to LDS
    uint32_t carry = 0u;
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const uint32_t incl = wave_scan_incl<Op::Add>((uint32_t)__builtin_popcount(m[j]));
      pre[j] = carry + wave_shift_excl<Op::Add>(incl);
      carry += readlane(incl, kWave - 1);
    }
    if (lane == 0) {
      post_wave_total<Op::Add, uint32_t, WD>(carry, wave, tile, s_wave, &s_posted, &s_agg_done,
                                             desc);
    }
  } else {
    // 2'. the look-back wave: walks back from the start and, once the last
    //     data wave has published the tile's count, publishes the tile's
    //     inclusive count and hands over the output offset
    auto tile_count = [&]() {
      uint32_t a = 0u;
#pragma unroll
      for (int w = 0; w < WD; ++w) a += s_wave[w];
      return a;
    };
    uint32_t prefix = 0u;
    if (tile > 0) {
      // fallback for a late predecessor: count its selected flags
      auto reduce_tile = [&](int64_t t) -> uint32_t {
        uint32_t acc = 0u;
        for (int c = 0; c < WD; ++c) {
          const int64_t first = t * kTileVecs + c * kWaveVecs;
          uint32_t g[K];
          load_flags(first, g);
          uint32_t cnt = 0u;
#pragma unroll
          for (int j = 0; j < K; ++j) cnt += (uint32_t)__builtin_popcount(select_mask(first + j * kWave, g[j]));
          acc += readlane(wave_scan_incl<Op::Add>(cnt), kWave - 1);
        }
        return acc;
      };
      prefix = look_back<Op::Add, uint32_t, kPollLong>(desc, tile, kLookBackTimeout, reduce_tile);
    }
    while (!lds_flag_set(&s_agg_done)) __builtin_amdgcn_s_sleep(1);
    if (lane == 0) {
      const uint32_t agg = tile_count();
      Desc<uint32_t>::publish(desc, tile, kInc, prefix + agg);
      s_prefix = prefix;
      if (tile == ntiles - 1) *num_out = (int32_t)(prefix + agg);
    }
  }
  __syncthreads();

  // 3. pack the selected elements into LDS, then store the run with 16-byte vectors
  const int64_t g = (int64_t)s_prefix;                 // output offset of this tile
  uint32_t before = 0u, count = 0u;
#pragma unroll
  for (int w = 0; w < WD; ++w) {
    const uint32_t c = s_wave[w];
    before += (w < wave) ? c : 0u;
    count += c;
  }
  const int s0 = (int)((g + out_ph) % EO);             // slot of the first selected element
  if (wave < WD) {
#pragma unroll
    for (int j = 0; j < K; ++j) {
      uint32_t r = (uint32_t)s0 + before + pre[j];
#pragma unroll
      for (int k = 0; k < E; ++k) {
        if ((m[j] >> k) & 1u) s_stage[r++] = x[j][k];
      }
    }
  }
  __syncthreads();
  const int64_t gv0 = (g + out_ph) / EO;               // first output vector of the run
  const int end = s0 + (int)count;
  const int nvec = (end + EO - 1) / EO;
  for (int w = (int)threadIdx.x; w < nvec; w += kThreads) {
    const int slot0 = w * EO;
    const uintptr_t dst = out_base + (uintptr_t)(gv0 + w) * 16;
    if (slot0 >= s0 && slot0 + EO <= end) {
      __builtin_nontemporal_store(*(const u32x4*)&s_stage[slot0], gptr<u32x4>(dst));
    } else {
#pragma unroll
      for (int k = 0; k < EO; ++k) {
        const int slot = slot0 + k;
        if (slot >= s0 && slot < end) *gptr<T>(dst + (uintptr_t)k * EB) = s_stage[slot];
      }
    }
  }
}

// Tiles of tv vectors covering window elements [ph, n + ph) (ph < e).
static int64_t sel_tiles_for(int64_t n, int e, int64_t tv) {
  if (n <= 0) return 0;
  const int64_t v_last = (n - 1 + (e - 1)) / e;
  return v_last / tv + 1;
}

// Sized for 8-byte elements (two per vector, the most tiles) and the smallest
// tile, so one scratch size serves both element widths and every launch shape.
size_t select_tiles(int64_t n, size_t elem_bytes) {
  (void)elem_bytes;
  return (size_t)sel_tiles_for(n, 2, kSelMinTileVecs);
}

__global__ void store_count_zero_kernel(int32_t* num_out) { *num_out = 0; }

// One launch shape: WD data waves (plus the look-back wave), K vectors per
// lane per tile.
template <int EB, int WD, int K>
static hipError_t launch_sel_cfg(const void* in, const uint8_t* flags, void* out, int32_t* num_out,
                                 int64_t n, void* scratch, hipStream_t stream,
                                 const int32_t* n_dev) {
  constexpr int E = 16 / EB;
  constexpr int64_t TV = (int64_t)kWave * WD * K;
  const uintptr_t ia = (uintptr_t)in, fa = (uintptr_t)flags, oa = (uintptr_t)out;
  const int64_t ph = (int64_t)((ia % 16) / EB);
  const int64_t out_ph = (int64_t)((oa % 16) / EB);
  const uintptr_t fbase = fa - (uintptr_t)ph;          // flag byte of window element 0
  const bool fvec = (fbase % E) == 0;
  const int64_t ntiles = sel_tiles_for(n, E, TV);
  uint64_t* desc = desc_base(scratch);
  hipError_t err = launch_fill_desc(desc, ntiles, Desc<uint32_t>::kWords, stream);
  if (err != hipSuccess) return err;
  const dim3 grid((unsigned)ntiles), block(64 * (WD + 1));
  const uintptr_t ibase = ia - (uintptr_t)ph * EB, obase = oa - (uintptr_t)out_ph * EB;
  if (fvec) {
    select_kernel<EB, E, true, WD, K><<<grid, block, 0, stream>>>(
        ibase, fbase, obase, n, n_dev, ph, out_ph, num_out, desc);
  } else {
    select_kernel<EB, E, false, WD, K><<<grid, block, 0, stream>>>(
        ibase, fbase, obase, n, n_dev, ph, out_ph, num_out, desc);
  }
  return hipGetLastError();
}

// Launch shape measured on MI355X over 2^28 f32 elements (us at p = 0.01 /
// 0.5 / 0.99): 3 data waves x 12 loads, staged through 48 KiB of LDS,
// 402 / 466 / 556; 3 x 16: 426 / 486 / 537; 7 x 8: 468 / 510 / 597.  Storing
// straight from registers instead of staging wins at low selectivity (328 us
// at p = 0.01) but loses at high (620 us at p = 0.99), so stores are staged.
template <int EB>
static hipError_t launch_sel_t(const void* in, const uint8_t* flags, void* out, int32_t* num_out,
                               int64_t n, void* scratch, hipStream_t stream,
                               const int32_t* n_dev) {
  return launch_sel_cfg<EB, 3, 12>(in, flags, out, num_out, n, scratch, stream, n_dev);
}

hipError_t launch_select(const void* in, const uint8_t* flags, void* out, int32_t* num_out,
                         int64_t n, size_t elem_bytes, void* scratch, hipStream_t stream,
                         const int32_t* n_dev) {
  if (n == 0) {
    store_count_zero_kernel<<<dim3(1), dim3(1), 0, stream>>>(num_out);
    return hipGetLastError();
  }
  if (elem_bytes == 4) return launch_sel_t<4>(in, flags, out, num_out, n, scratch, stream, n_dev);
  return launch_sel_t<8>(in, flags, out, num_out, n, scratch, stream, n_dev);
}

}  // namespace sca
