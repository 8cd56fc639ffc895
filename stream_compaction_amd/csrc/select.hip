// Stream compaction ("Algorithms" page, Quadrants user guide, section
// qd.algorithms.select): the flagged elements, in input order, become the
// dense prefix out[0..k) and k goes to num_out[0].
//
// The page's own realization is three phases (exclusive scan of the flags
// into an n-entry index buffer, scatter, one-thread count; section "Under the
// hood").  Here one kernel does all of it in a single pass, with the scan of
// the flag counts done by the same DPP wave scan and decoupled look-back as
// the device-wide scan, and no index buffer:
//   1. each lane loads 16-byte payload vectors (load j of lane l is vector
//      j*64 + l of its wave's segment) and the matching flag bytes, and forms
//      a bit mask of its selected elements;
//   2. lane counts are scanned across the wave (DPP), wave totals across the
//      workgroup (LDS), and the tile count across tiles (look-back), giving
//      the tile's output offset G; the tile with the last id writes num_out;
//   3. selected elements are packed into LDS at their rank, shifted so LDS
//      vectors line up with 16-byte vectors of `out`, and the workgroup
//      stores the packed run [G, G + count) with 16-byte stores (element
//      stores only for the partial vectors at its two ends).
// Elements move as raw bits, so any 4- or 8-byte type (NaN payloads
// included) is copied exactly.  out past the count is never written.
#include "device.hpp"
#include "launch.hpp"

namespace sca {

constexpr int kSelK = 8;                                   // vectors per lane per tile
constexpr int64_t kSelTileVecs = (int64_t)kBlock * kSelK;  // vectors per tile

template <int EB> struct Bits;
template <> struct Bits<4> { using T = uint32_t; };
template <> struct Bits<8> { using T = uint64_t; };

template <int EB, int E, bool FVEC, int K>
__global__ __launch_bounds__(256) void select_kernel(uintptr_t in_base, uintptr_t flags_base,
                                                    uintptr_t out_base, int64_t n, int64_t ph,
                                                    int64_t out_ph, int64_t ntiles,
                                                    int32_t* num_out, uint32_t* counter,
                                                    uint64_t* desc) {
  using T = typename Bits<EB>::T;
  constexpr int EO = 16 / EB;                     // elements per 16-byte output vector
  constexpr int64_t kTileVecs = (int64_t)kBlock * K;
  constexpr int kTileElems = (int)kTileVecs * E;
  __shared__ __attribute__((aligned(16))) T s_stage[kTileElems + EO];
  __shared__ uint32_t s_wave[kBlock / kWave];
  __shared__ uint32_t s_prefix;
  __shared__ int64_t s_tile;

  const int lane = lane_id(), wave = wave_id();
  if (threadIdx.x == 0)
    s_tile = (int64_t)__hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int64_t tile = s_tile;
  if (tile >= ntiles) return;

  const int64_t lo = ph, hi = n + ph, v_last = (hi - 1) / E;
  const int64_t vb = tile * kTileVecs + (int64_t)wave * kWave * K;

  // 1. payload and selection masks
  T x[K][E];
  uint32_t m[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const int64_t v = vb + j * kWave + lane;
    m[j] = 0u;
    if (v <= v_last) {
      const int64_t e0 = v * E;
      if (e0 >= lo && e0 + E <= hi) {
        if constexpr (E == 1) {
          x[j][0] = *(const T*)(in_base + e0 * EB);
        } else {
          const uint4 r = *(const uint4*)(in_base + e0 * EB);
          if constexpr (EB == 4) {
            x[j][0] = r.x; x[j][1] = r.y; x[j][2] = r.z; x[j][3] = r.w;
          } else {
            x[j][0] = ((uint64_t)r.y << 32) | r.x;
            x[j][1] = ((uint64_t)r.w << 32) | r.z;
          }
        }
        uint32_t f;
        if constexpr (FVEC && E == 4) {
          f = *(const uint32_t*)(flags_base + e0);
        } else if constexpr (FVEC && E == 2) {
          f = *(const uint16_t*)(flags_base + e0);
        } else {
          f = 0u;
#pragma unroll
          for (int k = 0; k < E; ++k) f |= (uint32_t)(*(const uint8_t*)(flags_base + e0 + k)) << (8 * k);
        }
#pragma unroll
        for (int k = 0; k < E; ++k) m[j] |= (((f >> (8 * k)) & 0xffu) != 0u ? 1u : 0u) << k;
      } else {
#pragma unroll
        for (int k = 0; k < E; ++k) {
          const int64_t i = e0 + k;
          if (i >= lo && i < hi) {
            x[j][k] = *(const T*)(in_base + i * EB);
            m[j] |= (*(const uint8_t*)(flags_base + i) != 0 ? 1u : 0u) << k;
          }
        }
      }
    }
  }

  // 2. ranks: within the wave, across waves, across tiles
  uint32_t pre[K];
  uint32_t carry = 0u;
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const uint32_t incl = wave_scan_incl<Op::Add>((uint32_t)__builtin_popcount(m[j]));
    pre[j] = carry + wave_shift_excl<Op::Add>(incl);
    carry += readlane(incl, kWave - 1);
  }
  if (lane == 0) s_wave[wave] = carry;
  __syncthreads();
  if (wave == 0) {
    uint32_t agg = 0u;
#pragma unroll
    for (int w = 0; w < kBlock / kWave; ++w) agg += s_wave[w];
    uint32_t prefix = 0u;
    if (tile == 0) {
      if (lane == 0) Desc<uint32_t>::publish(desc, tile, kInc, agg);
    } else {
      if (lane == 0) Desc<uint32_t>::publish(desc, tile, kAgg, agg);
      prefix = look_back<Op::Add, uint32_t>(desc, tile);
      if (lane == 0) Desc<uint32_t>::publish(desc, tile, kInc, prefix + agg);
    }
    if (lane == 0) {
      s_prefix = prefix;
      if (tile == ntiles - 1) *num_out = (int32_t)(prefix + agg);
    }
  }
  __syncthreads();

  // 3. pack into LDS, then store the run with 16-byte vectors
  const int64_t g = (int64_t)s_prefix;                 // output offset of this tile
  const int s0 = (int)((g + out_ph) % EO);             // slot of the first selected element
  uint32_t before = 0u, count = 0u;
#pragma unroll
  for (int w = 0; w < kBlock / kWave; ++w) {
    const uint32_t c = s_wave[w];
    before += (w < wave) ? c : 0u;
    count += c;
  }
#pragma unroll
  for (int j = 0; j < K; ++j) {
    uint32_t r = (uint32_t)s0 + before + pre[j];
#pragma unroll
    for (int k = 0; k < E; ++k) {
      if ((m[j] >> k) & 1u) s_stage[r++] = x[j][k];
    }
  }
  __syncthreads();
  const int64_t gv0 = (g + out_ph) / EO;               // first output vector of the run
  const int end = s0 + (int)count;
  const int nvec = (end + EO - 1) / EO;
  for (int w = (int)threadIdx.x; w < nvec; w += kBlock) {
    const int slot0 = w * EO;
    const uintptr_t dst = out_base + (uintptr_t)(gv0 + w) * 16;
    if (slot0 >= s0 && slot0 + EO <= end) {
      *(uint4*)dst = *(const uint4*)&s_stage[slot0];
    } else {
#pragma unroll
      for (int k = 0; k < EO; ++k) {
        const int slot = slot0 + k;
        if (slot >= s0 && slot < end) *(T*)(dst + (uintptr_t)k * EB) = s_stage[slot];
      }
    }
  }
}

static int64_t sel_tiles_for(int64_t n, int e) {
  if (n <= 0) return 0;
  const int64_t v_last = (n - 1 + (e - 1)) / e;
  return v_last / kSelTileVecs + 1;
}

// Sized for 8-byte elements (two per vector, the most tiles) so one scratch
// size serves both element widths.
size_t select_tiles(int64_t n, size_t elem_bytes) {
  (void)elem_bytes;
  return (size_t)sel_tiles_for(n, 2);
}

__global__ void store_count_zero_kernel(int32_t* num_out) { *num_out = 0; }

template <int EB>
static hipError_t launch_sel_t(const void* in, const uint8_t* flags, void* out, int32_t* num_out,
                               int64_t n, void* scratch, hipStream_t stream) {
  constexpr int E = 16 / EB;
  const uintptr_t ia = (uintptr_t)in, fa = (uintptr_t)flags, oa = (uintptr_t)out;
  const int64_t ph = (int64_t)((ia % 16) / EB);
  const int64_t out_ph = (int64_t)((oa % 16) / EB);
  const uintptr_t fbase = fa - (uintptr_t)ph;          // flag byte of window element 0
  const bool fvec = (fbase % E) == 0;
  const int64_t ntiles = sel_tiles_for(n, E);
  uint32_t* counter = (uint32_t*)scratch;
  uint64_t* desc = (uint64_t*)((char*)scratch + kScratchHeader);
  hipError_t err = launch_fill_zero(scratch, kScratchHeader + (size_t)ntiles * 8, stream);
  if (err != hipSuccess) return err;
  const dim3 grid((unsigned)ntiles), block(kBlock);
  const uintptr_t ibase = ia - (uintptr_t)ph * EB, obase = oa - (uintptr_t)out_ph * EB;
  if (fvec) {
    select_kernel<EB, E, true, kSelK><<<grid, block, 0, stream>>>(
        ibase, fbase, obase, n, ph, out_ph, ntiles, num_out, counter, desc);
  } else {
    select_kernel<EB, E, false, kSelK><<<grid, block, 0, stream>>>(
        ibase, fbase, obase, n, ph, out_ph, ntiles, num_out, counter, desc);
  }
  return hipGetLastError();
}

hipError_t launch_select(const void* in, const uint8_t* flags, void* out, int32_t* num_out,
                         int64_t n, size_t elem_bytes, void* scratch, hipStream_t stream) {
  if (n == 0) {
    store_count_zero_kernel<<<dim3(1), dim3(1), 0, stream>>>(num_out);
    return hipGetLastError();
  }
  if (elem_bytes == 4) return launch_sel_t<4>(in, flags, out, num_out, n, scratch, stream);
  return launch_sel_t<8>(in, flags, out, num_out, n, scratch, stream);
}

}  // namespace sca
