// Device-wide exclusive scan (add/min/max) in one pass over the data
// ("Algorithms" page, Quadrants user guide: section
// qd.algorithms.exclusive_scan_{add,min,max} for the contract, "Related" for
// decoupled look-back as the alternative to a phase-per-launch staircase).
//
// Each 256-thread workgroup takes the next tile id from an atomic counter (so
// every tile it may wait on belongs to a workgroup that is already running),
// loads its tile as 16-byte vectors (load j of lane l is vector j*64 + l of
// its wave's segment), and:
//   1. scans every vector lane-serially, then the 64 lane totals with a DPP
//      wave scan, keeping per vector the combine of everything before it in
//      the wave;
//   2. publishes the four wave totals through LDS; wave 0 forms the tile
//      aggregate, publishes it, looks back over predecessor descriptors to
//      get the tile's exclusive prefix, and publishes its inclusive prefix;
//   3. after one more barrier every lane combines tile prefix, earlier waves,
//      earlier vectors and earlier elements of its vector, and stores.
// The input is read once and the output written once.
#include "device.hpp"
#include "launch.hpp"

namespace sca {

constexpr int kDevK = 16;                                  // vectors per lane per tile
constexpr int64_t kDevTileVecs = (int64_t)kBlock * kDevK;  // vectors per tile

template <class F, Op O, int E, int K>
__global__ __launch_bounds__(256) void scan_device_kernel(uintptr_t in_base, uintptr_t out_base,
                                                         int64_t n, int64_t ph, int64_t ntiles,
                                                         uint32_t* counter, uint64_t* desc) {
  using S = typename F::S;
  using W = typename F::W;
  using IO = VecIO<S, E>;
  constexpr int64_t kTileVecs = (int64_t)kBlock * K;
  __shared__ W s_wave[kBlock / kWave];
  __shared__ W s_prefix;
  __shared__ int64_t s_tile;

  const int lane = lane_id(), wave = wave_id();
  if (threadIdx.x == 0)
    s_tile = (int64_t)__hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int64_t tile = s_tile;
  if (tile >= ntiles) return;

  const W id = identity<O, W>();
  const int64_t lo = ph, hi = n + ph, v_last = (hi - 1) / E;
  const int64_t vb = tile * kTileVecs + (int64_t)wave * kWave * K;

  typename IO::Raw raw[K];
  const S id_s = narrow<F>(id);
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const int64_t v = vb + j * kWave + lane;
    raw[j] = (v <= v_last) ? IO::load(in_base, v, lo, hi, id_s) : typename IO::Raw{};
  }
  W x[K][E];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const int64_t v = vb + j * kWave + lane;
    if (v <= v_last) {
      IO::template unpack<F>(raw[j], x[j]);
    } else {
#pragma unroll
      for (int k = 0; k < E; ++k) x[j][k] = id;
    }
  }

  // 1. within the wave
  W pre[K];
  W carry = id;
#pragma unroll
  for (int j = 0; j < K; ++j) {
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
    for (int w = 1; w < kBlock / kWave; ++w) agg = combine<O>(agg, s_wave[w]);
    W prefix = id;
    if (tile == 0) {
      if (lane == 0) Desc<W>::publish(desc, tile, kInc, agg);
    } else {
      if (lane == 0) Desc<W>::publish(desc, tile, kAgg, agg);
      prefix = look_back<O, W>(desc, tile);
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
    const int64_t v = vb + j * kWave + lane;
    if (v <= v_last) IO::template store<F>(out_base, v, lo, hi, y);
  }
}

// Tiles covering window elements [ph, n + ph) (ph < e) in vectors of e elements.
static int64_t tiles_for(int64_t n, int e) {
  if (n <= 0) return 0;
  const int64_t v_last = (n - 1 + (e - 1)) / e;
  return v_last / kDevTileVecs + 1;
}

static int fmt_bytes(Fmt f) {
  switch (f) {
    case Fmt::F16: case Fmt::BF16: return 2;
    case Fmt::F64: case Fmt::I64: case Fmt::U64: return 8;
    default: return 4;
  }
}

size_t scan_device_desc_words(Fmt fmt) { return fmt_bytes(fmt) == 8 ? 4 : 1; }

// Sized for the slowest path (one element per vector) so one scratch size
// serves every pointer alignment.
size_t scan_device_tiles(int64_t n, Fmt fmt) {
  (void)fmt;
  return (size_t)tiles_for(n, 1);
}

template <class F, Op O>
static hipError_t launch_dev_t(const void* in, void* out, int64_t n, void* scratch,
                               hipStream_t stream) {
  using S = typename F::S;
  constexpr int EV = 16 / (int)sizeof(S);
  const uintptr_t ia = (uintptr_t)in, oa = (uintptr_t)out;
  uint32_t* counter = (uint32_t*)scratch;
  uint64_t* desc = (uint64_t*)((char*)scratch + kScratchHeader);
  const bool vec = (ia % 16) == (oa % 16);
  const int e = vec ? EV : 1;
  const int64_t ph = vec ? (int64_t)((ia % 16) / sizeof(S)) : 0;
  const int64_t ntiles = tiles_for(n, e);
  hipError_t err = launch_fill_zero(
      scratch, kScratchHeader + (size_t)ntiles * Desc<typename F::W>::kWords * 8, stream);
  if (err != hipSuccess) return err;
  const dim3 grid((unsigned)ntiles), block(kBlock);
  if (vec) {
    scan_device_kernel<F, O, EV, kDevK><<<grid, block, 0, stream>>>(
        ia - ph * sizeof(S), oa - ph * sizeof(S), n, ph, ntiles, counter, desc);
  } else {
    scan_device_kernel<F, O, 1, kDevK><<<grid, block, 0, stream>>>(ia, oa, n, 0, ntiles, counter,
                                                                    desc);
  }
  return hipGetLastError();
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
