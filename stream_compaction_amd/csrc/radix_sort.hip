// Stable LSD radix sort of 32- or 64-bit keys, optionally carrying values
// ("Algorithms" page, Quadrants user guide, section qd.algorithms.sort:
// ascending, stable, 8-bit digits, keys mapped to a sortable unsigned image;
// each digit pass is a tile histogram, a scan of the digit-major histogram
// buffer, and a scatter).  Per pass, on tiles whose size depends on the key
// and value widths (RxShape below: 8,192 keys for 32-bit keys alone or with
// 8-byte values, 16,384 for 32-bit keys with 4-byte values, 4,096 for 64-bit
// keys alone and 8,192 for 64-bit keys with values):
//   1. radix_tile_hist_kernel: every tile counts its keys per digit (per-wave
//      LDS counters) and writes the 256 counts digit-major,
//      hist[d * ntiles + t];
//   2. the library's own device-wide exclusive scan turns that buffer into
//      each (digit, tile)'s first output position: all keys with a smaller
//      digit, plus the keys with this digit in earlier tiles;
//   3. radix_scatter_kernel: every tile ranks its keys stably within the
//      tile - for each load, the lanes holding the same digit are found
//      through a per-wave LDS table of lane masks, and a lane's rank is the
//      count of such lanes below it plus the wave's running count of that
//      digit, so ranks follow input order - reorders them by digit in LDS,
//      and writes every digit's run contiguously at its output position;
//      values follow the same permutation.
// Both per-tile kernels hand each XCD a contiguous range of tiles.
// A single-pass variant with a per-digit decoupled look-back (one read of the
// keys per pass instead of two) was measured slower on MI355X: with ~500
// tiles resident, each digit's walk waited on predecessors that were still
// ranking, and wider look-back windows flooded the memory system with polls.
// Sortable image: unsigned keys as they are; signed keys with the sign bit
// flipped; floats with the sign bit flipped when clear and all bits flipped
// when set (-0 before +0); every NaN takes the largest image (NaNs last, in
// input order, as the page states for numpy.sort).  Only the low end_bit bits
// of the image are sorted on.  Keys and values move as raw bits.
#include "device.hpp"
#include "launch.hpp"

namespace sca {

enum class KeyKind : int { Unsigned, Signed, Float };

template <class KT, KeyKind KK>
__device__ __forceinline__ KT sort_image(KT k) {
  constexpr KT top = KT(1) << (sizeof(KT) * 8 - 1);
  if constexpr (KK == KeyKind::Unsigned) {
    return k;
  } else if constexpr (KK == KeyKind::Signed) {
    return k ^ top;
  } else {
    constexpr KT inf = sizeof(KT) == 4 ? KT(0x7f800000u) : KT(0x7ff0000000000000ull);
    if ((k & ~top) > inf) return ~KT(0);          // NaN of either sign: last
    return (k & top) ? ~k : (k | top);
  }
}

constexpr int kRxBins = 256;

// Workgroups are handed to the eight XCDs in turn (workgroup b to XCD b % 8).
// This mapping gives each XCD a contiguous range of tiles, taken in order, so
// what neighbouring tiles write side by side (their histogram counts, the
// pieces of a digit's output run) meets in one L2 and leaves it as whole
// lines.
__device__ __forceinline__ int64_t rx_xcd_tile(int64_t b, int64_t ntiles) {
  const int64_t q = ntiles / 8, r = ntiles % 8, x = b % 8, i = b / 8;
  return x * q + (x < r ? x : r) + i;
}
// ---------------------------------------------------------------------------
// 2. one digit pass
// ---------------------------------------------------------------------------

// ---------------------------------------------------------------------------
// 1. tile histograms, digit-major
// ---------------------------------------------------------------------------
// It also zeroes the descriptors of the device scan that follows it on the
// stream (workgroup b clears descriptors b, b + grid, ...), so that scan needs
// no fill kernel of its own.
template <class KT, KeyKind KK, int WAVES, int KPT>
__global__ __launch_bounds__(64 * WAVES) void radix_tile_hist_kernel(
    const KT* __restrict__ kin, int64_t n_cap, const int32_t* n_dev, int shift, int64_t ntiles,
    uint32_t* hist, uint64_t* scan_desc, int64_t scan_ndesc) {
  constexpr int kThreads = 64 * WAVES;
  constexpr int kTile = kThreads * KPT;
  __shared__ uint32_t s_h[WAVES][kRxBins];
  const int tid = threadIdx.x, wave = wave_id();
  if (tid == 0) {
    for (int64_t d = blockIdx.x; d < scan_ndesc; d += gridDim.x) scan_desc[d * kDescLineWords] = 0ull;
  }
  const int64_t tile = rx_xcd_tile(blockIdx.x, ntiles);
  const int64_t t0 = tile * kTile;
  const int64_t n = live_count(n_cap, n_dev);
  const int count = (int)((n - t0) < kTile ? ((n - t0) > 0 ? (n - t0) : 0) : kTile);
  for (int i = tid; i < WAVES * kRxBins; i += kThreads) (&s_h[0][0])[i] = 0u;
  __syncthreads();
  // 16-byte loads through a buffer resource bounded at the tile's last key
  // (the order of the keys does not matter to a histogram)
  constexpr int kE = 16 / (int)sizeof(KT);            // keys per 16-byte vector
  constexpr int kLoads = KPT / kE;
  const Buf buf((uintptr_t)(kin + t0), (int64_t)count * (int64_t)sizeof(KT));
  u32x4 r[kLoads];
#pragma unroll
  for (int j = 0; j < kLoads; ++j)
    r[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
        buf.r, (uint32_t)(((j * kThreads + tid) * kE) * (int)sizeof(KT)), 0, kNT));
  auto count_keys = [&](auto full) {
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
#pragma unroll
      for (int e = 0; e < kE; ++e) {
        const int s = (j * kThreads + tid) * kE + e;
        KT key;
        if constexpr (sizeof(KT) == 4) {
          key = r[j][e];
        } else {
          key = ((KT)r[j][2 * e + 1] << 32) | r[j][2 * e];
        }
        if (decltype(full)::value || s < count) {
          const uint32_t d = (uint32_t)((sort_image<KT, KK>(key) >> shift) & 255u);
          __hip_atomic_fetch_add(&s_h[wave][d], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
      }
    }
  };
  if (count == kTile) {
    count_keys(std::true_type{});
  } else {
    count_keys(std::false_type{});
  }
  __syncthreads();
  for (int d = tid; d < kRxBins; d += kThreads) {
    uint32_t h = 0u;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) h += s_h[w][d];
    hist[(int64_t)d * ntiles + tile] = h;
  }
}

// ---------------------------------------------------------------------------
// 3. rank, reorder and scatter one tile
// ---------------------------------------------------------------------------
template <int VB> struct ValBits { using T = uint32_t; };
template <> struct ValBits<8> { using T = uint64_t; };

// Ranking history, measured on MI355X.  An earlier full-wave form kept the
// whole wave's 64-bit lane mask in the table entry and the running count in a
// separate per-wave array: fewer LDS instructions than the half-wave form
// (below), but more registers.  The half-wave form pays wherever the
// registers it frees let more workgroups share a CU.  Keys only: 2.78
// against 3.06 ms for 2^28 u32 keys.  With values, together with the late
// value loads and packed positions (below) and tiles of 16 waves: 32-bit keys
// with 4-byte values 4.64 against 5.22 ms (2^28 pairs), with 8-byte values
// 6.94 against 7.48 ms; 64-bit keys with 4- / 8-byte values 7.60 / 9.61
// against 8.28 / 10.66 ms (2^27 pairs).  Without those (values held through
// the ranking, one workgroup per CU, or 8-wave tiles) it had lost: 5.36-5.41
// against 5.24 ms, and 9.14 / 11.79 against 8.31 / 10.69 ms.

// A buffer resource over [base, base + bytes) for bytes < 2^32: offsets are
// 32-bit, and accesses past the range read zero or are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rx_rsrc(const void* base, uint64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)(uint32_t)bytes, 0x00020000);
}
template <class T>
__device__ __forceinline__ T rx_load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (sizeof(T) == 4) {
    return (T)__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kNT);
  } else {
    return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kNT));
  }
}
template <class T>
__device__ __forceinline__ void rx_store(__amdgpu_buffer_rsrc_t r, uint32_t off, T x) {
  if constexpr (sizeof(T) == 4) {
    __builtin_amdgcn_raw_buffer_store_b32((uint32_t)x, r, off, 0, 0);
  } else {
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, x), r, off, 0, 0);
  }
}

// Ranking.  For each load, the lanes holding the same digit are found through
// a per-wave LDS table, one 64-bit entry per digit (and one for "no key"):
// the lanes of a half-wave OR their bit into the entry's low word, read the
// entry back and write it with the mask cleared and the high word, the
// wave's running count of the digit, advanced.  LDS work from one wave is
// carried out in issue order, so a read sees the OR of every lane of its half
// and the next half's or load's ORs come after the write.  A lane's rank is
// the count of matching lanes below it in its half plus the running count, so
// ranks follow input order.
//
// Stores: with B32 the outputs are written through buffer resources with
// 32-bit byte offsets (every array below 4 GiB); else through 64-bit
// addresses.  FULL tiles skip every per-key range test.
template <class KT, KeyKind KK, int VB, int WAVES, int KPT, bool B32, bool FULL>
__device__ __forceinline__ void rx_scatter_tile(
    const KT* __restrict__ kin, KT* __restrict__ kout, const void* __restrict__ vin_,
    void* __restrict__ vout_, int64_t n, int shift, int64_t t0, int count,
    uint16_t (*s_wcnt)[kRxBins + 1], uint32_t* s_start, uint32_t* s_g, uint32_t* s_sum,
    unsigned char* s_buf) {
  using VT = typename ValBits<VB>::T;
  constexpr int kThreads = 64 * WAVES;
  constexpr int kBins1 = kRxBins + 1;                // digit 256: no key
  KT* s_keys = (KT*)s_buf;
  VT* s_vals = (VT*)s_buf;
  uint64_t* s_tab = (uint64_t*)s_buf + wave_id() * kBins1;   // this wave's lane-mask table
  const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();

  // With values, the values are loaded only once
  // the keys are ranked, and ranks, reorder positions and output digits are
  // held packed (two or four to a register).  That brings the 16-wave
  // workgroups with values to 41-60 VGPRs, so two share a CU.
  constexpr bool kLateV = VB != 0;

  // ---- load (buffer resources bounded at the tile's keys) ----
  const int wbase = wave * 64 * KPT;                 // the wave's first slot in the tile
  const auto kr = rx_rsrc(kin + t0, (uint64_t)count * sizeof(KT));
  KT k[KPT];
  VT v[VB != 0 ? KPT : 1];
#pragma unroll
  for (int j = 0; j < KPT; ++j) k[j] = rx_load<KT>(kr, (uint32_t)((wbase + j * 64 + lane) * sizeof(KT)));
  auto load_values = [&]() {
    const auto vr = rx_rsrc((const VT*)vin_ + t0, (uint64_t)count * VB);
    // the lane's first offset, opaque to the compiler: the loads then take
    // j * 64 * VB as their immediate offset instead of sixteen address
    // registers computed ahead of time
    uint32_t vo = (uint32_t)((wbase + lane) * VB);
    if constexpr (kLateV) asm volatile("" : "+v"(vo));
#pragma unroll
    for (int j = 0; j < KPT; ++j) v[j] = rx_load<VT>(vr, vo + (uint32_t)(j * 64 * VB));
  };
  auto valid = [&](int j) { return FULL || wbase + j * 64 + lane < count; };
  uint32_t dg[KPT], rank[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    dg[j] = (uint32_t)((sort_image<KT, KK>(k[j]) >> shift) & 255u);
    if constexpr (!FULL) dg[j] = wbase + j * 64 + lane < count ? dg[j] : (uint32_t)kRxBins;
  }

  // ---- rank within the wave ----
  // Each table entry holds, in its low word, the lane mask of one half-wave
  // for the current load and, in its high word, the wave's running count of
  // the digit.  The lower half of the wave goes first: its lanes OR in their
  // bits, read the entry (mask and count), and write back a clear mask with
  // the count advanced; the upper half then does the same and so sees the
  // lower half's keys counted, which keeps ranks in input order.
  const uint16_t* cnt = s_wcnt[wave];                // each digit's first slot, after the prefix phase
  const uint32_t hbit = 1u << (lane & 31);
  uint32_t rpk[(KPT + 1) / 2] = {};                  // ranks, two 16-bit halves a register
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    uint64_t* e = s_tab + dg[j];
    uint32_t r = 0u;
    if (lane < 32) {
      __hip_atomic_fetch_or((uint32_t*)e, hbit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      const uint64_t t = __hip_atomic_load(e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      const uint32_t m = (uint32_t)t, c = (uint32_t)(t >> 32);
      // every lane of the digit writes the same entry
      __hip_atomic_store(e, (uint64_t)(c + (uint32_t)__builtin_popcount(m)) << 32,
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      r = c + __builtin_amdgcn_mbcnt_lo(m, 0u);
    }
    if (lane >= 32) {
      __hip_atomic_fetch_or((uint32_t*)e, hbit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      const uint64_t t = __hip_atomic_load(e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      const uint32_t m = (uint32_t)t, c = (uint32_t)(t >> 32);
      __hip_atomic_store(e, (uint64_t)(c + (uint32_t)__builtin_popcount(m)) << 32,
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      r = c + __builtin_amdgcn_mbcnt_hi(m, 0u);
    }
    if constexpr (kLateV) {
      rpk[j >> 1] |= r << ((j & 1) * 16);            // below the tile size
    } else {
      rank[j] = r;
    }
  }
  __syncthreads();

  // ---- per digit: each wave's first slot in the tile ----
  if (tid < kRxBins) {
    uint32_t h = 0u;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      const uint32_t c = (uint32_t)(((const uint64_t*)s_buf)[w * kBins1 + tid] >> 32);
      s_wcnt[w][tid] = (uint16_t)h;
      h += c;
    }
    const uint32_t incl = wave_scan_incl<Op::Add>(h);
    if (lane == kWave - 1) s_sum[wave] = incl;
    s_start[tid] = incl - h;                          // within this wave of digits, for now
  }
  __syncthreads();
  if (tid < kRxBins) {
    uint32_t off = 0u;
    for (int w = 0; w < wave; ++w) off += s_sum[w];
    const uint32_t st = s_start[tid] + off;           // the digit's first slot in the tile
    s_g[tid] -= st;                                   // its output position minus that slot
#pragma unroll
    for (int w = 0; w < WAVES; ++w) s_wcnt[w][tid] = (uint16_t)(s_wcnt[w][tid] + st);
  }
  __syncthreads();

  // ---- reorder by digit in LDS (the tables are no longer needed) ----
  if constexpr (kLateV) load_values();             // in flight while the keys move
  int lpos[KPT];
  uint32_t lpk[(KPT + 1) / 2] = {};                  // kLateV: positions, two a register
  // kLateV: the shift and the keys made opaque here, so the digits (and the
  // keys' sortable images) are computed again rather than held across the
  // barriers
  int sh = shift;
  if constexpr (kLateV) {
    asm volatile("" : "+s"(sh));
#pragma unroll
    for (int j = 0; j < KPT; ++j) asm volatile("" : "+v"(k[j]));
  }
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    if constexpr (kLateV) {
      // the digit again from the key, the rank from its packed half
      const uint32_t d = valid(j) ? (uint32_t)((sort_image<KT, KK>(k[j]) >> sh) & 255u)
                                  : (uint32_t)kRxBins;
      const uint32_t p = (uint32_t)cnt[d] + ((rpk[j >> 1] >> ((j & 1) * 16)) & 0xffffu);
      lpk[j >> 1] |= (p & 0xffffu) << ((j & 1) * 16);
      if (valid(j)) s_keys[p] = k[j];
    } else {
      lpos[j] = (int)((uint32_t)cnt[dg[j]] + rank[j]);
      if (FULL || dg[j] < (uint32_t)kRxBins) s_keys[lpos[j]] = k[j];
    }
  }
  __syncthreads();

  // ---- write every digit's run in place ----
  // (positions are below n by construction; the range checks only keep every
  // store inside the output whatever the input)
  const auto okr = rx_rsrc(kout, B32 ? (uint64_t)n * sizeof(KT) : 0);
  uint32_t dpk[(KPT + 3) / 4] = {};                  // kLateV: each slot's digit, four a register
#pragma unroll
  for (int m = 0; m < KPT; ++m) {
    const int slot = tid + m * kThreads;
    if (FULL || slot < count) {
      const KT key = s_keys[slot];
      const uint32_t d = (uint32_t)((sort_image<KT, KK>(key) >> shift) & 255u);
      const uint32_t g = s_g[d] + (uint32_t)slot;     // modulo 2^32, like the offsets
      if constexpr (kLateV) dpk[m >> 2] |= d << ((m & 3) * 8);
      if constexpr (B32) {
        rx_store<KT>(okr, g * (uint32_t)sizeof(KT), key);
      } else {
        if (g < (uint64_t)n) *gptr<KT>((uintptr_t)(kout + g)) = key;
      }
    }
    // kLateV: at most four slots' reads in flight, and each word of digits
    // packed as soon as it is whole, which bounds the registers
    if (kLateV && (m & 3) == 3) asm volatile("" : "+v"(dpk[m >> 2]) : : "memory");
  }
  if constexpr (VB != 0) {
    __syncthreads();                                   // every key is out of the buffer
    if constexpr (kLateV) {
      // opaque from here: unpacked only now, not kept unpacked through the key writes
#pragma unroll
      for (int i = 0; i < (KPT + 1) / 2; ++i) asm volatile("" : "+v"(lpk[i]));
#pragma unroll
      for (int i = 0; i < (KPT + 3) / 4; ++i) asm volatile("" : "+v"(dpk[i]));
    }
#pragma unroll
    for (int j = 0; j < KPT; ++j)
      if (valid(j)) s_vals[(lpk[j >> 1] >> ((j & 1) * 16)) & 0xffffu] = v[j];
    __syncthreads();
    VT* vout = (VT*)vout_;
    const auto ovr = rx_rsrc(vout, B32 ? (uint64_t)n * VB : 0);
#pragma unroll
    for (int m = 0; m < KPT; ++m) {
      const int slot = tid + m * kThreads;
      if (FULL || slot < count) {
        const VT x = s_vals[slot];
        const uint32_t g = s_g[(dpk[m >> 2] >> ((m & 3) * 8)) & 255u] + (uint32_t)slot;
        if constexpr (B32) {
          rx_store<VT>(ovr, g * (uint32_t)VB, x);
        } else {
          if (g < (uint64_t)n) *gptr<VT>((uintptr_t)(vout + g)) = x;
        }
      }
      if ((m & 3) == 3) asm volatile("" ::: "memory");
    }
  }
}

template <class KT, KeyKind KK, int VB, int WAVES, int KPT, bool B32>
__global__ __launch_bounds__(64 * WAVES) void radix_scatter_kernel(
    const KT* __restrict__ kin, KT* __restrict__ kout, const void* __restrict__ vin,
    void* __restrict__ vout, int64_t n_cap, const int32_t* n_dev, int shift, int64_t ntiles,
    const uint32_t* __restrict__ offsets) {
  constexpr int kThreads = 64 * WAVES;
  constexpr int kTile = kThreads * KPT;
  constexpr int kBins1 = kRxBins + 1;
  constexpr int kSortBytes = kTile * (int)(sizeof(KT) > (size_t)VB ? sizeof(KT) : (size_t)VB);
  constexpr int kTabBytes = WAVES * kBins1 * 8;
  // the digits' first slots sit past the tables until the reorder
  constexpr int kTabStartBytes = kTabBytes + kRxBins * 4;
  constexpr int kBufBytes = kSortBytes > kTabStartBytes ? kSortBytes : kTabStartBytes;
  static_assert(kThreads >= kRxBins, "one thread per digit");
  // The running counts live in the lane-mask tables; this array only holds
  // each wave's first slot per digit, below the tile size: 16 bits, which
  // keeps a keys-only workgroup under a quarter of the CU's LDS (four
  // resident instead of three).
  static_assert(kTile < 65536, "first slots fit 16 bits");
  __shared__ uint16_t s_wcnt[WAVES][kBins1];    // per wave: each digit's first slot
  __shared__ uint32_t s_g[kRxBins];             // the digit's first output position (then
                                                // that minus its first slot in the tile)
  __shared__ uint32_t s_sum[kRxBins / 64];
  // lane-mask tables while ranking, then the tile reordered by digit
  __shared__ __attribute__((aligned(16))) unsigned char s_buf[kBufBytes];
  uint32_t* s_start = (uint32_t*)(s_buf + kTabBytes);   // the digit's first slot in the tile

  const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
  const int64_t tile = rx_xcd_tile(blockIdx.x, ntiles);
  const int64_t t0 = tile * kTile;
  const int64_t n = live_count(n_cap, n_dev);
  const int count =                                  // keys in this tile
      (int)((n - t0) < kTile ? ((n - t0) > 0 ? (n - t0) : 0) : kTile);
  uint64_t* tab = (uint64_t*)s_buf + wave * kBins1;
  for (int i = lane; i < kBins1; i += kWave) tab[i] = 0ull;
  if (tid < kRxBins) s_g[tid] = offsets[(int64_t)tid * ntiles + tile];
  __syncthreads();
  if (count == kTile) {
    rx_scatter_tile<KT, KK, VB, WAVES, KPT, B32, true>(kin, kout, vin, vout, n, shift, t0, count,
                                                       s_wcnt, s_start, s_g, s_sum, s_buf);
  } else {
    rx_scatter_tile<KT, KK, VB, WAVES, KPT, B32, false>(kin, kout, vin, vout, n, shift, t0, count,
                                                        s_wcnt, s_start, s_g, s_sum, s_buf);
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void rx_copy_kernel(const uint4* src, uint4* dst, int64_t n16) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256)
    dst[i] = src[i];
}

__global__ void rx_copy_tail_kernel(const unsigned char* src, unsigned char* dst, int64_t bytes) {
  for (int64_t i = threadIdx.x; i < bytes; i += blockDim.x) dst[i] = src[i];
}

static unsigned grid_for(int64_t items, int64_t per_block, int64_t cap) {
  int64_t g = (items + per_block - 1) / per_block;
  if (g < 1) g = 1;
  if (g > cap) g = cap;
  return (unsigned)g;
}

static hipError_t rx_copy(const void* src, void* dst, size_t bytes, hipStream_t stream) {
  // both buffers are element aligned; copy 16-byte vectors when they share a phase
  if (((uintptr_t)src % 16) == ((uintptr_t)dst % 16)) {
    const size_t head = (16 - (uintptr_t)src % 16) % 16;
    const size_t h = head < bytes ? head : bytes;
    if (h) rx_copy_tail_kernel<<<1, 64, 0, stream>>>((const unsigned char*)src, (unsigned char*)dst, (int64_t)h);
    const int64_t n16 = (int64_t)((bytes - h) / 16);
    if (n16) {
      rx_copy_kernel<<<grid_for(n16, 256, 4096), 256, 0, stream>>>(
          (const uint4*)((const unsigned char*)src + h), (uint4*)((unsigned char*)dst + h), n16);
    }
    const size_t done = h + (size_t)n16 * 16;
    if (done < bytes) {
      rx_copy_tail_kernel<<<1, 256, 0, stream>>>((const unsigned char*)src + done,
                                                 (unsigned char*)dst + done,
                                                 (int64_t)(bytes - done));
    }
  } else {
    const int64_t nb = (int64_t)bytes;
    rx_copy_tail_kernel<<<1, 1024, 0, stream>>>((const unsigned char*)src, (unsigned char*)dst, nb);
  }
  return hipGetLastError();
}

// Tile shape per key and value width.  32-bit keys alone: 8 waves x 16 keys
// per thread (8192 keys; 16 x 16 cost the keys-only sort its occupancy, 5.31
// against 4.19 ms in an earlier version).  With values, 16 waves (two
// workgroups per CU, 74,800 bytes of LDS each, the reorder buffer holding one
// tile of the wider of key and value): 16 x 16 (16384 keys) for 32-bit keys
// with 4-byte values, 16 x 8 (8192) for 8-byte values and for 64-bit keys.
// Longer digit runs halve the write streams per key: 16 x 16 measured 7.40
// against 8.79 ms for 2^28 key-value pairs in an earlier version, and 8 x 16
// measures 6.32 against 4.66 ms now.  64-bit keys alone: 8 waves x 8.
template <class KT, int VB> struct RxShape { static constexpr int kWaves = 8, kKpt = 8; };
template <> struct RxShape<uint32_t, 0> { static constexpr int kWaves = 8, kKpt = 16; };
template <> struct RxShape<uint32_t, 4> { static constexpr int kWaves = 16, kKpt = 16; };
template <> struct RxShape<uint32_t, 8> { static constexpr int kWaves = 16, kKpt = 8; };
template <> struct RxShape<uint64_t, 4> { static constexpr int kWaves = 16, kKpt = 8; };
template <> struct RxShape<uint64_t, 8> { static constexpr int kWaves = 16, kKpt = 8; };

template <class KT, int VB>
constexpr int64_t rx_tile() {
  return (int64_t)64 * RxShape<KT, VB>::kWaves * RxShape<KT, VB>::kKpt;
}

// The histogram kernel's shape: 16-byte loads per lane over the scatter's
// tile.  Measured per pass over 2^28 u32 keys (tiles of 8,192 / 16,384):
// 4 loads 180 / 174 us, 8 loads 186 / 179, 16 loads 197 / 186.
#ifndef SCA_RX_HIST_LOADS
#define SCA_RX_HIST_LOADS 4
#endif
template <class KT, int VB> struct RxHistShape {
  static constexpr int kKpt = SCA_RX_HIST_LOADS * (16 / (int)sizeof(KT));
  static constexpr int kWaves = (int)(rx_tile<KT, VB>() / (64 * kKpt));
  static_assert(kWaves >= 1 && (int64_t)kWaves * 64 * kKpt == rx_tile<KT, VB>(),
                "the histogram covers the scatter's tile");
};

// Scratch layout: the digit-major tile histograms (ntiles * 256 u32), their
// exclusive scan (the same size), then the device-wide scan's own scratch.
// Sized for the smallest tile of the key width, so one size serves every
// value width.
static int64_t rx_ntiles(int64_t n, int64_t tile) { return (n + tile - 1) / tile; }
static int64_t rx_min_tile(size_t key_bytes) {
  if (key_bytes == 8) {
    const int64_t a = rx_tile<uint64_t, 0>(), b = rx_tile<uint64_t, 4>(), c = rx_tile<uint64_t, 8>();
    const int64_t m = a < b ? a : b;
    return m < c ? m : c;
  }
  const int64_t a = rx_tile<uint32_t, 0>(), b = rx_tile<uint32_t, 4>(), c = rx_tile<uint32_t, 8>();
  const int64_t m = a < b ? a : b;
  return m < c ? m : c;
}

static size_t rx_hist_bytes(int64_t ntiles) {
  return ((size_t)ntiles * kRxBins * 4 + 15) & ~(size_t)15;
}

size_t radix_sort_scratch(int64_t n, size_t key_bytes) {
  if (n <= 1) return 0;
  const int64_t nt = rx_ntiles(n, rx_min_tile(key_bytes));
  return 2 * rx_hist_bytes(nt) + desc_scratch_bytes(scan_device_tiles(nt * kRxBins, Fmt::U32));
}

template <class KT, KeyKind KK, int VB>
static hipError_t launch_rx_t(void* keys, void* tmp_keys, void* values, void* tmp_values, int64_t n,
                              int end_bit, void* scratch, hipStream_t stream,
                              const int32_t* n_dev) {
  constexpr int W = RxShape<KT, VB>::kWaves, KPT = RxShape<KT, VB>::kKpt;
  const int npass = end_bit / 8;
  // with a device count the result must land in `keys` by itself (an even
  // number of passes): a copy back would need the count on the host
  if (n_dev != nullptr && npass % 2 == 1) return hipErrorInvalidValue;
  const int64_t ntiles = rx_ntiles(n, rx_tile<KT, VB>());
  uint32_t* hist = (uint32_t*)scratch;
  uint32_t* offs = (uint32_t*)((char*)scratch + rx_hist_bytes(ntiles));
  void* scan_scratch = (char*)scratch + 2 * rx_hist_bytes(ntiles);
  // the histogram kernel clears the scan's descriptors (one word each)
  static_assert(Desc<uint32_t>::kWords == 1, "one descriptor word per tile");
  uint64_t* const scan_desc = desc_base(scan_scratch);
  const int64_t scan_ndesc = (int64_t)scan_device_tiles(ntiles * kRxBins, Fmt::U32);
  KT* src = (KT*)keys;
  KT* dst = (KT*)tmp_keys;
  void* vsrc = values;
  void* vdst = tmp_values;
  // every key and value array below 4 GiB: 32-bit buffer offsets for the scatter
  const bool b32 = (uint64_t)n * (sizeof(KT) > (size_t)VB ? sizeof(KT) : (size_t)VB) < (1ull << 32);
  hipError_t err = hipSuccess;
  for (int p = 0; p < npass; ++p) {
    constexpr int HW = RxHistShape<KT, VB>::kWaves, HKPT = RxHistShape<KT, VB>::kKpt;
    radix_tile_hist_kernel<KT, KK, HW, HKPT><<<dim3((unsigned)ntiles), dim3(64 * HW), 0, stream>>>(
        src, n, n_dev, 8 * p, ntiles, hist, scan_desc, scan_ndesc);
    err = hipGetLastError();
    if (err == hipSuccess)
      err = launch_scan_device(hist, offs, ntiles * kRxBins, Fmt::U32, 0, false, scan_scratch,
                               stream, nullptr, true);
    if (err != hipSuccess) return err;
    if (b32) {
      radix_scatter_kernel<KT, KK, VB, W, KPT, true><<<dim3((unsigned)ntiles), dim3(64 * W), 0, stream>>>(
          src, dst, vsrc, vdst, n, n_dev, 8 * p, ntiles, offs);
    } else {
      radix_scatter_kernel<KT, KK, VB, W, KPT, false><<<dim3((unsigned)ntiles), dim3(64 * W), 0, stream>>>(
          src, dst, vsrc, vdst, n, n_dev, 8 * p, ntiles, offs);
    }
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    KT* ts = src; src = dst; dst = ts;
    void* tv = vsrc; vsrc = vdst; vdst = tv;
  }
  if (npass % 2 == 1) {                       // the result is in the temporaries: copy it back
    err = rx_copy(tmp_keys, keys, (size_t)n * sizeof(KT), stream);
    if (err == hipSuccess && VB != 0) err = rx_copy(tmp_values, values, (size_t)n * VB, stream);
  }
  return err;
}

template <class KT, KeyKind KK>
static hipError_t launch_rx_v(void* keys, void* tmp_keys, void* values, void* tmp_values, int64_t n,
                              int value_bytes, int end_bit, void* scratch, hipStream_t stream,
                              const int32_t* n_dev) {
  switch (value_bytes) {
    case 0: return launch_rx_t<KT, KK, 0>(keys, tmp_keys, nullptr, nullptr, n, end_bit, scratch, stream, n_dev);
    case 4: return launch_rx_t<KT, KK, 4>(keys, tmp_keys, values, tmp_values, n, end_bit, scratch, stream, n_dev);
    default: return launch_rx_t<KT, KK, 8>(keys, tmp_keys, values, tmp_values, n, end_bit, scratch, stream, n_dev);
  }
}

hipError_t launch_radix_sort(void* keys, void* tmp_keys, void* values, void* tmp_values, int64_t n,
                             Fmt kfmt, int value_bytes, int end_bit, void* scratch,
                             hipStream_t stream, const int32_t* n_dev) {
  if (n <= 1) return hipSuccess;
  switch (kfmt) {
    case Fmt::U32: return launch_rx_v<uint32_t, KeyKind::Unsigned>(keys, tmp_keys, values, tmp_values, n, value_bytes, end_bit, scratch, stream, n_dev);
    case Fmt::I32: return launch_rx_v<uint32_t, KeyKind::Signed>(keys, tmp_keys, values, tmp_values, n, value_bytes, end_bit, scratch, stream, n_dev);
    case Fmt::F32: return launch_rx_v<uint32_t, KeyKind::Float>(keys, tmp_keys, values, tmp_values, n, value_bytes, end_bit, scratch, stream, n_dev);
    case Fmt::U64: return launch_rx_v<uint64_t, KeyKind::Unsigned>(keys, tmp_keys, values, tmp_values, n, value_bytes, end_bit, scratch, stream, n_dev);
    case Fmt::I64: return launch_rx_v<uint64_t, KeyKind::Signed>(keys, tmp_keys, values, tmp_values, n, value_bytes, end_bit, scratch, stream, n_dev);
    case Fmt::F64: return launch_rx_v<uint64_t, KeyKind::Float>(keys, tmp_keys, values, tmp_values, n, value_bytes, end_bit, scratch, stream, n_dev);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sca
