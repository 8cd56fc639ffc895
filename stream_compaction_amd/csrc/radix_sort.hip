// Stable LSD radix sort of 32- or 64-bit keys, optionally carrying values
// ("Algorithms" page, Quadrants user guide, section qd.algorithms.sort:
// ascending, stable, 8-bit digits, keys mapped to a sortable unsigned image;
// each digit pass is a tile histogram, a scan of the digit-major histogram
// buffer, and a scatter).  Per pass, on tiles of 8192 (32-bit keys) or 4096
// (64-bit keys) keys:
//   1. radix_tile_hist_kernel: every tile counts its keys per digit (per-wave
//      LDS counters) and writes the 256 counts digit-major,
//      hist[d * ntiles + t];
//   2. the library's own device-wide exclusive scan turns that buffer into
//      each (digit, tile)'s first output position: all keys with a smaller
//      digit, plus the keys with this digit in earlier tiles;
//   3. radix_scatter_kernel: every tile ranks its keys stably within the
//      tile - for each load, the lanes holding the same digit are found with
//      eight ballots (one per digit bit), and a lane's rank is the count of
//      such lanes below it plus the wave's running count of that digit (kept
//      in LDS), so ranks follow input order - reorders them by digit in LDS,
//      and writes every digit's run contiguously at its output position;
//      values follow the same permutation.
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
// ---------------------------------------------------------------------------
// 2. one digit pass
// ---------------------------------------------------------------------------

// ---------------------------------------------------------------------------
// 1. tile histograms, digit-major
// ---------------------------------------------------------------------------
template <class KT, KeyKind KK, int WAVES, int KPT>
__global__ __launch_bounds__(64 * WAVES) void radix_tile_hist_kernel(
    const KT* __restrict__ kin, int64_t n_cap, const int32_t* n_dev, int shift, int64_t ntiles,
    uint32_t* hist) {
  constexpr int kThreads = 64 * WAVES;
  constexpr int kTile = kThreads * KPT;
  static_assert(kThreads >= kRxBins, "one thread per digit");
  __shared__ uint32_t s_h[WAVES][kRxBins];
  const int tid = threadIdx.x, wave = wave_id();
  const int64_t tile = blockIdx.x;
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
      if (s < count) {
        const uint32_t d = (uint32_t)((sort_image<KT, KK>(key) >> shift) & 255u);
        __hip_atomic_fetch_add(&s_h[wave][d], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
    }
  }
  __syncthreads();
  if (tid < kRxBins) {
    uint32_t h = 0u;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) h += s_h[w][tid];
    hist[(int64_t)tid * ntiles + tile] = h;
  }
}

// ---------------------------------------------------------------------------
// 3. rank, reorder and scatter one tile
// ---------------------------------------------------------------------------
template <int VB> struct ValBits { using T = uint32_t; };
template <> struct ValBits<8> { using T = uint64_t; };

template <class KT, KeyKind KK, int VB, int WAVES, int KPT>
__global__ __launch_bounds__(64 * WAVES) void radix_scatter_kernel(
    const KT* __restrict__ kin, KT* __restrict__ kout, const void* __restrict__ vin_,
    void* __restrict__ vout_, int64_t n_cap, const int32_t* n_dev, int shift, int64_t ntiles,
    const uint32_t* __restrict__ offsets) {
  using VT = typename ValBits<VB>::T;
  constexpr int kThreads = 64 * WAVES;
  constexpr int kTile = kThreads * KPT;
  constexpr int kBufBytes = kTile * (int)(sizeof(KT) > (size_t)VB ? sizeof(KT) : (size_t)VB);
  static_assert(kThreads >= kRxBins, "one thread per digit");
  __shared__ uint32_t s_wcnt[WAVES][kRxBins];   // per wave: running count, then exclusive prefix
  __shared__ uint32_t s_start[kRxBins];         // the digit's first slot in the tile
  __shared__ uint32_t s_g[kRxBins];             // the digit's first output position (then
                                                // that minus its first slot in the tile)
  __shared__ uint32_t s_sum[4];
  __shared__ __attribute__((aligned(16))) unsigned char s_buf[kBufBytes];
  KT* s_keys = (KT*)s_buf;
  VT* s_vals = (VT*)s_buf;
  const VT* vin = (const VT*)vin_;
  VT* vout = (VT*)vout_;

  const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
  const int64_t tile = blockIdx.x;
  const int64_t t0 = tile * kTile;
  const int64_t n = live_count(n_cap, n_dev);
  const int count =                                  // keys in this tile
      (int)((n - t0) < kTile ? ((n - t0) > 0 ? (n - t0) : 0) : kTile);
  for (int i = tid; i < WAVES * kRxBins; i += kThreads) (&s_wcnt[0][0])[i] = 0u;
  if (tid < kRxBins) s_g[tid] = offsets[(int64_t)tid * ntiles + tile];
  __syncthreads();

  // ---- load, and rank within the wave (stable: ranks follow input order) ----
  const int wbase = wave * 64 * KPT;                 // the wave's first slot in the tile
  KT k[KPT];
  VT v[VB != 0 ? KPT : 1];
  uint32_t dg[KPT], rank[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int s = wbase + j * 64 + lane;
    k[j] = s < count ? *gptr<const KT>((uintptr_t)(kin + t0 + s)) : KT(0);
    if constexpr (VB != 0) v[j] = s < count ? *gptr<const VT>((uintptr_t)(vin + t0 + s)) : VT(0);
  }
#pragma unroll
  for (int j = 0; j < KPT; ++j)
    dg[j] = wbase + j * 64 + lane < count
                ? (uint32_t)((sort_image<KT, KK>(k[j]) >> shift) & 255u) : 256u;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const bool valid = dg[j] < 256u;
    // lanes whose digit equals this lane's: for each digit bit, keep the
    // lanes that agree with it, match &= ~(ballot ^ sext(bit)), as one
    // three-input bit operation per 32-bit half (gfx950 v_bitop3_b32)
    const uint64_t v = __ballot(valid);
    uint32_t mlo = (uint32_t)v, mhi = (uint32_t)(v >> 32);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const uint32_t sx = (uint32_t)__builtin_amdgcn_sbfe((int)dg[j], b, 1);   // 0 or ~0
      const uint64_t bb = __ballot(sx != 0u);
      // 0x90 is the truth table of a & ~(b ^ c) over operands (a, b, c)
      mlo = __builtin_amdgcn_bitop3_b32(mlo, (uint32_t)bb, sx, 0x90);
      mhi = __builtin_amdgcn_bitop3_b32(mhi, (uint32_t)(bb >> 32), sx, 0x90);
    }
    const uint64_t match = ((uint64_t)mhi << 32) | mlo;
    const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(match >> 32),
                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)match, 0u));
    const uint32_t same = (uint32_t)__builtin_popcountll(match);
    const uint32_t old = valid ? s_wcnt[wave][dg[j]] : 0u;
    if (valid && below == 0u) s_wcnt[wave][dg[j]] = old + same;
    rank[j] = old + below;
  }
  __syncthreads();

  // ---- per digit: prefix over waves, and the digit's first slot in the tile ----
  if (tid < kRxBins) {
    uint32_t h = 0u;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      const uint32_t c = s_wcnt[w][tid];
      s_wcnt[w][tid] = h;
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
    s_start[tid] += off;
    // the digit's output position minus its first slot in the tile
    s_g[tid] -= s_start[tid];
  }
  __syncthreads();

  // ---- reorder by digit in LDS, then write every digit's run in place ----
  int lpos[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    lpos[j] = -1;
    if (dg[j] < 256u) {
      lpos[j] = (int)(s_start[dg[j]] + s_wcnt[wave][dg[j]] + rank[j]);
      s_keys[lpos[j]] = k[j];
    }
  }
  __syncthreads();
  // (positions are below n by construction; the bound only keeps every store
  // inside the output whatever the input)
  int32_t dst[KPT];
#pragma unroll
  for (int m = 0; m < KPT; ++m) {
    const int slot = tid + m * kThreads;
    dst[m] = -1;
    if (slot < count) {
      const KT key = s_keys[slot];
      const uint32_t d = (uint32_t)((sort_image<KT, KK>(key) >> shift) & 255u);
      const uint32_t g = s_g[d] + (uint32_t)slot;     // modulo 2^32, like the offsets
      if (g < (uint64_t)n) {
        dst[m] = (int32_t)g;
        *gptr<KT>((uintptr_t)(kout + g)) = key;
      }
    }
  }
  if constexpr (VB != 0) {
    __syncthreads();                                   // every key is out of the buffer
#pragma unroll
    for (int j = 0; j < KPT; ++j)
      if (lpos[j] >= 0) s_vals[lpos[j]] = v[j];
    __syncthreads();
#pragma unroll
    for (int m = 0; m < KPT; ++m)
      if (dst[m] >= 0) *gptr<VT>((uintptr_t)(vout + dst[m])) = s_vals[tid + m * kThreads];
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
// per thread (8192 keys).  32-bit keys with 4-byte values: 16 waves x 16
// (16384 keys, one workgroup per CU by LDS): the longer digit runs halve the
// write streams per key, which measured 7.40 ms against 8.79 ms for 2^28
// key-value pairs, while costing the keys-only sort (5.31 ms against 4.19)
// its occupancy.  32-bit keys with 8-byte values: 8 x 16.  64-bit keys: 8
// waves x 8 (the LDS reorder buffer holds one tile of the wider of key and
// value).
template <class KT, int VB> struct RxShape { static constexpr int kWaves = 8, kKpt = 8; };
template <> struct RxShape<uint32_t, 0> { static constexpr int kWaves = 8, kKpt = 16; };
template <> struct RxShape<uint32_t, 4> { static constexpr int kWaves = 16, kKpt = 16; };
template <> struct RxShape<uint32_t, 8> { static constexpr int kWaves = 8, kKpt = 16; };

template <class KT, int VB>
constexpr int64_t rx_tile() {
  return (int64_t)64 * RxShape<KT, VB>::kWaves * RxShape<KT, VB>::kKpt;
}

// Scratch layout: the digit-major tile histograms (ntiles * 256 u32), their
// exclusive scan (the same size), then the device-wide scan's own scratch.
// Sized for the smallest tile of the key width, so one size serves every
// value width.
static int64_t rx_ntiles(int64_t n, int64_t tile) { return (n + tile - 1) / tile; }
static int64_t rx_min_tile(size_t key_bytes) {
  if (key_bytes == 8) return rx_tile<uint64_t, 0>();
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
  KT* src = (KT*)keys;
  KT* dst = (KT*)tmp_keys;
  void* vsrc = values;
  void* vdst = tmp_values;
  hipError_t err = hipSuccess;
  for (int p = 0; p < npass; ++p) {
    radix_tile_hist_kernel<KT, KK, W, KPT><<<dim3((unsigned)ntiles), dim3(64 * W), 0, stream>>>(
        src, n, n_dev, 8 * p, ntiles, hist);
    err = hipGetLastError();
    if (err == hipSuccess)
      err = launch_scan_device(hist, offs, ntiles * kRxBins, Fmt::U32, 0, false, scan_scratch,
                               stream);
    if (err != hipSuccess) return err;
    radix_scatter_kernel<KT, KK, VB, W, KPT><<<dim3((unsigned)ntiles), dim3(64 * W), 0, stream>>>(
        src, dst, vsrc, vdst, n, n_dev, 8 * p, ntiles, offs);
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
