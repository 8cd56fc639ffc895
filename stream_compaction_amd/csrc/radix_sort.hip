// Stable LSD radix sort of 32- or 64-bit keys, optionally carrying values
// ("Algorithms" page, Quadrants user guide, section qd.algorithms.sort:
// ascending, stable, 8-bit digits, keys mapped to a sortable unsigned image).
//
// The page runs three kernels per digit pass (tile histograms, a scan of the
// digit-major histogram buffer, scatter), reading the keys twice per pass.
// Here the digit histograms of every pass come from ONE read of the keys up
// front, and each pass is ONE kernel that reads its keys once and writes
// them once:
//   1. radix_hist_kernel: global digit counts of every pass (LDS counters,
//      then one atomic add per nonzero bin); radix_bases_kernel turns them
//      into each digit's first output position (exclusive scan over digits).
//   2. radix_pass_kernel, per pass: workgroup b owns tile b of the input.
//      - Its waves load their keys (load j of lane l is key j*64 + l of the
//        wave's run) and rank them: for each load, the lanes holding the same
//        digit are found with eight ballots (one per digit bit), a lane's
//        rank is the count of such lanes below it plus the wave's running
//        count of that digit (kept in LDS), so ranks follow input order and
//        the sort is stable.
//      - Per digit, the tile's count is published at once, and one thread
//        per digit walks back over the predecessors' per-digit descriptors
//        (decoupled look-back, as in the device-wide scan) to find how many
//        keys with that digit come before the tile; it then publishes the
//        inclusive count.
//      - Keys are reordered by digit in LDS (stable), then written so that
//        every digit's run lands contiguously at its global position; values
//        follow the same permutation.
// Sortable image: unsigned keys as they are; signed keys with the sign bit
// flipped; floats with the sign bit flipped when clear and all bits flipped
// when set (-0 before +0); every NaN takes the largest image (NaNs last, in
// input order, as the page states for numpy.sort).  Only the low end_bit bits
// of the image are sorted on.  Keys and values move as raw bits.
//
// Descriptor words are 32-bit: status in the top two bits, count in the low
// thirty, so n < 2^30.  Pass p uses descriptor array p % 2 and clears, tile by
// tile, the other array for pass p + 1; array 0 is cleared before pass 0.
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

constexpr uint32_t kRxNone = 0u, kRxAgg = 1u, kRxInc = 2u;
constexpr uint32_t kRxCountMask = (1u << 30) - 1u;
constexpr int kRxBins = 256;

__device__ __forceinline__ void rx_store(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t rx_load(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// 1. digit histograms of every pass, and each digit's first output position
// ---------------------------------------------------------------------------
template <class KT, KeyKind KK>
__global__ __launch_bounds__(256) void radix_hist_kernel(const KT* __restrict__ keys, int64_t n,
                                                         int npass, uint32_t* ghist) {
  __shared__ uint32_t s_h[8 * kRxBins];
  for (int i = threadIdx.x; i < npass * kRxBins; i += 256) s_h[i] = 0u;
  __syncthreads();
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const KT img = sort_image<KT, KK>(keys[i]);
    for (int p = 0; p < npass; ++p)
      __hip_atomic_fetch_add(&s_h[p * kRxBins + (int)((img >> (8 * p)) & 255u)], 1u,
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < npass * kRxBins; i += 256) {
    const uint32_t c = s_h[i];
    if (c) __hip_atomic_fetch_add(&ghist[i], c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// One workgroup per pass: base[p][d] = sum of ghist[p][d'] over d' < d.
__global__ __launch_bounds__(256) void radix_bases_kernel(const uint32_t* ghist, uint32_t* base) {
  __shared__ uint32_t s_w[4];
  const int d = threadIdx.x, lane = lane_id(), wave = wave_id();
  const uint32_t c = ghist[blockIdx.x * kRxBins + d];
  const uint32_t incl = wave_scan_incl<Op::Add>(c);
  if (lane == kWave - 1) s_w[wave] = incl;
  __syncthreads();
  uint32_t off = 0u;
  for (int w = 0; w < wave; ++w) off += s_w[w];
  base[blockIdx.x * kRxBins + d] = off + incl - c;
}

// ---------------------------------------------------------------------------
// 2. one digit pass
// ---------------------------------------------------------------------------
template <int VB> struct ValBits { using T = uint32_t; };
template <> struct ValBits<8> { using T = uint64_t; };

template <class KT, KeyKind KK, int VB, int WAVES, int KPT>
__global__ __launch_bounds__(64 * WAVES) void radix_pass_kernel(
    const KT* __restrict__ kin, KT* __restrict__ kout, const void* __restrict__ vin_,
    void* __restrict__ vout_, int64_t n, int shift, const uint32_t* __restrict__ base,
    uint32_t* desc, uint32_t* desc_next) {
  using VT = typename ValBits<VB>::T;
  constexpr int kThreads = 64 * WAVES;
  constexpr int kTile = kThreads * KPT;
  constexpr int kBufBytes = kTile * (int)(sizeof(KT) > (size_t)VB ? sizeof(KT) : (size_t)VB);
  static_assert(kThreads >= kRxBins, "one thread per digit");
  __shared__ uint32_t s_wcnt[WAVES][kRxBins];   // per wave: running count, then exclusive prefix
  __shared__ uint32_t s_start[kRxBins];         // the digit's first slot in the tile
  __shared__ uint32_t s_g[kRxBins];             // the digit's first output position
  __shared__ uint32_t s_sum[4];
  __shared__ __attribute__((aligned(16))) unsigned char s_buf[kBufBytes];
  KT* s_keys = (KT*)s_buf;
  VT* s_vals = (VT*)s_buf;
  const VT* vin = (const VT*)vin_;
  VT* vout = (VT*)vout_;

  const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
  const int64_t tile = blockIdx.x;
  const int64_t t0 = tile * kTile;
  const int count = (int)((n - t0) < kTile ? (n - t0) : kTile);   // keys in this tile
  if (desc_next != nullptr && tid < kRxBins) desc_next[tile * kRxBins + tid] = 0u;
  for (int i = tid; i < WAVES * kRxBins; i += kThreads) (&s_wcnt[0][0])[i] = 0u;
  __syncthreads();

  // ---- load, and rank within the wave (stable: ranks follow input order) ----
  const int wbase = wave * 64 * KPT;                 // the wave's first slot in the tile
  KT k[KPT];
  uint32_t dg[KPT], rank[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int s = wbase + j * 64 + lane;
    k[j] = s < count ? kin[t0 + s] : KT(0);
    dg[j] = s < count ? (uint32_t)((sort_image<KT, KK>(k[j]) >> shift) & 255u) : 256u;
  }
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const bool valid = dg[j] < 256u;
    uint64_t match = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const uint64_t bb = __ballot((dg[j] >> b) & 1u);
      match &= ((dg[j] >> b) & 1u) ? bb : ~bb;
    }
    const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(match >> 32),
                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)match, 0u));
    const uint32_t same = (uint32_t)__builtin_popcountll(match);
    const uint32_t old = valid ? s_wcnt[wave][dg[j]] : 0u;
    if (valid && below == 0u) s_wcnt[wave][dg[j]] = old + same;
    rank[j] = old + below;
  }
  __syncthreads();

  // ---- per digit: tile count, publish it, prefix over waves, slot starts ----
  uint32_t h = 0u;
  if (tid < kRxBins) {
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      const uint32_t c = s_wcnt[w][tid];
      s_wcnt[w][tid] = h;
      h += c;
    }
    rx_store(&desc[tile * kRxBins + tid], ((tile == 0 ? kRxInc : kRxAgg) << 30) | h);
    const uint32_t incl = wave_scan_incl<Op::Add>(h);
    if (lane == kWave - 1) s_sum[wave] = incl;
    s_start[tid] = incl - h;                          // within this wave of digits, for now
  }
  __syncthreads();
  if (tid < kRxBins) {
    uint32_t off = 0u;
    for (int w = 0; w < wave; ++w) off += s_sum[w];
    s_start[tid] += off;

    // ---- look-back for this digit ----
    uint32_t excl = 0u;
    if (tile > 0) {
      int64_t t = tile - 1;
      uint64_t tstart = __builtin_amdgcn_s_memrealtime();
      for (;;) {
        const uint32_t w = rx_load(&desc[t * kRxBins + tid]);
        const uint32_t st = w >> 30;
        if (st != kRxNone) {
          excl += w & kRxCountMask;
          if (st == kRxInc || t == 0) break;
          --t;
          tstart = __builtin_amdgcn_s_memrealtime();
          continue;
        }
        if (__builtin_amdgcn_s_memrealtime() - tstart > kLookBackTimeout) {
          // the predecessor has not published: count its keys with this digit
          const int64_t lo = t * kTile, hi = (n - lo) < kTile ? n : lo + kTile;
          uint32_t c = 0u;
          for (int64_t i = lo; i < hi; ++i)
            c += ((sort_image<KT, KK>(kin[i]) >> shift) & 255u) == (uint32_t)tid ? 1u : 0u;
          excl += c;
          if (t == 0) break;
          --t;
          tstart = __builtin_amdgcn_s_memrealtime();
          continue;
        }
        __builtin_amdgcn_s_sleep(kPollShort);
      }
      rx_store(&desc[tile * kRxBins + tid], (kRxInc << 30) | ((excl + h) & kRxCountMask));
    }
    s_g[tid] = base[tid] + excl;
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
  // (positions are below n < 2^30 by construction; the bound only keeps every
  // store inside the output whatever the input)
  int32_t dst[KPT];
#pragma unroll
  for (int m = 0; m < KPT; ++m) {
    const int slot = tid + m * kThreads;
    dst[m] = -1;
    if (slot < count) {
      const KT key = s_keys[slot];
      const uint32_t d = (uint32_t)((sort_image<KT, KK>(key) >> shift) & 255u);
      const int64_t g = (int64_t)s_g[d] + (slot - (int)s_start[d]);
      if (g >= 0 && g < n) {
        dst[m] = (int32_t)g;
        kout[g] = key;
      }
    }
  }
  if constexpr (VB != 0) {
    VT v[KPT];
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int s = wbase + j * 64 + lane;
      v[j] = s < count ? vin[t0 + s] : VT(0);
    }
    __syncthreads();                                   // every key is out of the buffer
#pragma unroll
    for (int j = 0; j < KPT; ++j)
      if (lpos[j] >= 0) s_vals[lpos[j]] = v[j];
    __syncthreads();
#pragma unroll
    for (int m = 0; m < KPT; ++m)
      if (dst[m] >= 0) vout[dst[m]] = s_vals[tid + m * kThreads];
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void rx_zero_kernel(uint4* p, int64_t n16) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256)
    p[i] = uint4{0u, 0u, 0u, 0u};
}

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

static hipError_t rx_zero(void* p, size_t bytes, hipStream_t stream) {
  const int64_t n16 = (int64_t)(bytes / 16);
  if (n16 == 0) return hipSuccess;
  rx_zero_kernel<<<grid_for(n16, 256, 4096), 256, 0, stream>>>((uint4*)p, n16);
  return hipGetLastError();
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

// Tile shape per key width: 8 waves; 16 keys per thread for 32-bit keys, 8 for
// 64-bit keys (the LDS reorder buffer holds one tile of the wider of key and
// value).
template <class KT> struct RxShape;
template <> struct RxShape<uint32_t> { static constexpr int kWaves = 8, kKpt = 16; };
template <> struct RxShape<uint64_t> { static constexpr int kWaves = 8, kKpt = 8; };

template <class KT>
constexpr int64_t rx_tile() {
  return (int64_t)64 * RxShape<KT>::kWaves * RxShape<KT>::kKpt;
}

// Scratch layout: ghist [8][256] u32, base [8][256] u32, then two descriptor
// arrays of ntiles * 256 u32 each, starting on a 128-byte boundary.
size_t radix_sort_scratch(int64_t n, size_t key_bytes) {
  if (n <= 0) return 0;
  const int64_t tile = key_bytes == 8 ? rx_tile<uint64_t>() : rx_tile<uint32_t>();
  const int64_t ntiles = (n + tile - 1) / tile;
  return (size_t)(2 * 8 * kRxBins * 4) + 128 + (size_t)ntiles * kRxBins * 4 * 2;
}

template <class KT, KeyKind KK, int VB>
static hipError_t launch_rx_t(void* keys, void* tmp_keys, void* values, void* tmp_values, int64_t n,
                              int end_bit, void* scratch, hipStream_t stream) {
  constexpr int W = RxShape<KT>::kWaves, KPT = RxShape<KT>::kKpt;
  constexpr int64_t kTile = rx_tile<KT>();
  const int npass = end_bit / 8;
  const int64_t ntiles = (n + kTile - 1) / kTile;
  uint32_t* ghist = (uint32_t*)scratch;
  uint32_t* base = ghist + 8 * kRxBins;
  uint32_t* d0 = (uint32_t*)((((uintptr_t)(base + 8 * kRxBins)) + 127) & ~(uintptr_t)127);
  uint32_t* d1 = d0 + ntiles * kRxBins;
  hipError_t err = rx_zero(ghist, (size_t)8 * kRxBins * 4, stream);
  if (err == hipSuccess) err = rx_zero(d0, (size_t)ntiles * kRxBins * 4, stream);
  if (err != hipSuccess) return err;
  radix_hist_kernel<KT, KK><<<grid_for(n, 256 * 16, 2048), 256, 0, stream>>>((const KT*)keys, n,
                                                                             npass, ghist);
  radix_bases_kernel<<<npass, 256, 0, stream>>>(ghist, base);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  KT* src = (KT*)keys;
  KT* dst = (KT*)tmp_keys;
  void* vsrc = values;
  void* vdst = tmp_values;
  for (int p = 0; p < npass; ++p) {
    uint32_t* dcur = (p % 2 == 0) ? d0 : d1;
    uint32_t* dnext = (p + 1 < npass) ? ((p % 2 == 0) ? d1 : d0) : nullptr;
    radix_pass_kernel<KT, KK, VB, W, KPT><<<dim3((unsigned)ntiles), dim3(64 * W), 0, stream>>>(
        src, dst, vsrc, vdst, n, 8 * p, base + p * kRxBins, dcur, dnext);
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
                              int value_bytes, int end_bit, void* scratch, hipStream_t stream) {
  switch (value_bytes) {
    case 0: return launch_rx_t<KT, KK, 0>(keys, tmp_keys, nullptr, nullptr, n, end_bit, scratch, stream);
    case 4: return launch_rx_t<KT, KK, 4>(keys, tmp_keys, values, tmp_values, n, end_bit, scratch, stream);
    default: return launch_rx_t<KT, KK, 8>(keys, tmp_keys, values, tmp_values, n, end_bit, scratch, stream);
  }
}

hipError_t launch_radix_sort(void* keys, void* tmp_keys, void* values, void* tmp_values, int64_t n,
                             Fmt kfmt, int value_bytes, int end_bit, void* scratch,
                             hipStream_t stream) {
  if (n <= 1) return hipSuccess;
  switch (kfmt) {
    case Fmt::U32: return launch_rx_v<uint32_t, KeyKind::Unsigned>(keys, tmp_keys, values, tmp_values, n, value_bytes, end_bit, scratch, stream);
    case Fmt::I32: return launch_rx_v<uint32_t, KeyKind::Signed>(keys, tmp_keys, values, tmp_values, n, value_bytes, end_bit, scratch, stream);
    case Fmt::F32: return launch_rx_v<uint32_t, KeyKind::Float>(keys, tmp_keys, values, tmp_values, n, value_bytes, end_bit, scratch, stream);
    case Fmt::U64: return launch_rx_v<uint64_t, KeyKind::Unsigned>(keys, tmp_keys, values, tmp_values, n, value_bytes, end_bit, scratch, stream);
    case Fmt::I64: return launch_rx_v<uint64_t, KeyKind::Signed>(keys, tmp_keys, values, tmp_values, n, value_bytes, end_bit, scratch, stream);
    case Fmt::F64: return launch_rx_v<uint64_t, KeyKind::Float>(keys, tmp_keys, values, tmp_values, n, value_bytes, end_bit, scratch, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sca
