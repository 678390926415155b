// Sliding-window attention prefill in IEEE fp32 (every product and sum in
// fp32: the fp32 workloads are held to an absolute error of 1e-5).
//
// Same definition as the bf16 kernel (robocikowo glossary "Sliding Window
// Attention", opening definition; Ultralytics glossary, section "Come cresce
// la finestra con la profondita"): each query row takes the softmax of its
// in-window logits only.
//
// One kernel on the matrix cores (prefill_f32_mfma_kernel below:
// v_mfma_f32_32x32x2_f32, the tiled bf16 kernel's decomposition) takes every
// mode: plain and dilated windows, the chunk continuing a ring cache, and the
// window plus global tokens (whose global rows the split-K pass of
// swa_ring.hip writes afterwards).

#include "swa_device.h"
#include "swa_launch.h"
#include "swa_tile_math.h"

namespace swa {
namespace {

// ---------------------------------------------------------------------------
// Plain and dilated windows, the chunk continuing a ring cache (Ultralytics
// ring-buffer paragraph) and the window plus global tokens (aivaro answer 629,
// sections 4.2 and 4.3), on the matrix cores.  The tiled bf16 kernel's
// decomposition: one workgroup = 128 query rows of one query head (of one
// residue class mod the dilation, a sequence of its own with row stride
// dil * d), four waves of 32 rows; 64-key K/V tiles visited only where they
// meet the block's windows, double-buffered in LDS and filled by direct
// buffer-to-LDS loads; S^T = K Q^T with one query row per lane.  Products on
// v_mfma_f32_32x32x2_f32; softmax exact and online per 32-key block (a
// reference maximum raised lazily, sums in fp32, probabilities
// exp2(s * c - m) with c = scale * log2(e)); O^T += V^T P^T with the fp32
// probabilities as they are.  The chunk mode
// (MODE 2) is the causal kernel in key coordinates relative to the chunk's
// first token at position p, as in the bf16 kernel: key r < 0 is position
// p + r, read from ring slot (p + r) mod W; tiles are aligned to the chunk
// start, so a tile is wholly ring or wholly chunk.  The global-token modes
// (MODES 5 causal, 6 symmetric, any dilation) visit the global keys after the
// window's tiles, as extra tiles whose rows are gathered from the global
// positions; a global key already inside a row's window, or after the row
// when causal, is masked there.
//
// The tile's two 32-key blocks are taken one after the other, each with its
// own online-softmax update.
//
// Operand layout.  A 32x32x2 product takes, in lane l, element l / 32 of its
// step's two-element slice of the reduced dimension.  S^T = K Q^T reduces
// over dims, assigned to (step, lane half) as d = 8 * (step / 4) + 4 * half +
// step % 4, so that a lane's operands of four consecutive steps are four
// consecutive floats: one 16-byte read of its Q row at the start, one of its
// K row per four steps.  O^T += V^T P^T reduces over keys: step j of a 32-key
// block takes key 8 * (j / 4) + 4 * half + j % 4, which is exactly score
// register j of the lane (the result layout of every 32x32 product), so the
// probabilities are the B operand with no data movement; V^T comes as single
// floats, V[key][32 * md + l % 32].
namespace f32m {

constexpr int kBN = tm::kBN;   // keys per tile
constexpr int kBM = tm::kBM;   // query rows per workgroup
constexpr int kThreads = 256;  // four waves
constexpr int kBufferFlags = 0x00020000;  // raw 32-bit buffer access

// log2 headroom of a row's probabilities over its reference maximum
constexpr float kGrow = 64.0f;

template <int D>
struct Geo {
  static constexpr int ROWB = D * 4;                   // bytes per K/V row in LDS
  static constexpr int TILEB = kBN * ROWB;             // bytes per tile
  static constexpr int NLD = TILEB / (kThreads * 16);  // direct loads per thread per tile
  static constexpr int KQ = D / 8;                     // 16-byte operand groups per lane
  static constexpr int MD = D / 32;                    // 32-dim output blocks
};

// XOR swizzle of a K row's 16-byte chunks: the K operand read (16 lanes, 16
// consecutive rows, one logical chunk) touches every bank group once.  V rows
// are stored as they are (its single-float reads, 32 consecutive floats of
// two rows, meet each bank at most twice), so that their addresses differ by
// constants and need no registers of their own.
template <int D>
__device__ __forceinline__ int swz(int row) {
  return D == 32 ? ((row >> 1) & 7) : (row & 15);
}

// Occupancy (waves per SIMD) that the LDS of double-buffered fp32 tiles
// allows: 128 KB per workgroup at d = 128, 64 KB at d = 64, 32 KB at d = 32
// (the chunk and global-token modes at d = 32 take three, whose registers
// hold their ring or global-key addressing without spills).
template <int D, int MODE>
constexpr int kWaves = D == 128 ? 1 : (D == 64 ? 2 : (MODE == 2 || MODE >= 5 ? 3 : 4));

}  // namespace f32m

// MODE: 0 causal, 1 symmetric (dil: key stride of a dilated window), 2 causal
// chunk continuing a ring cache (Tseq is then the chunk length; kring, vring,
// pos and hkv_seq are used by MODE 2 only), 5 causal and 6 symmetric window
// (dilated when dil > 1) plus the ngl global keys at gpos.
template <int D, int MODE>
__global__ __launch_bounds__(f32m::kThreads)
__attribute__((amdgpu_waves_per_eu(f32m::kWaves<D, MODE>, f32m::kWaves<D, MODE>)))
void prefill_f32_mfma_kernel(const float* __restrict__ q, const float* __restrict__ k,
                             const float* __restrict__ v, float* __restrict__ out, int Tseq,
                             int W, int Hq, int Hkv, float c, int n_qtiles, int dil,
                             const float* __restrict__ kring, const float* __restrict__ vring,
                             const int32_t* __restrict__ pos, int hkv_seq,
                             const int32_t* __restrict__ gpos, int ngl) {
  using namespace f32m;
  constexpr bool kCausal = MODE != 1 && MODE != 6;
  constexpr bool kChunk = MODE == 2;
  constexpr bool kGlobal = MODE >= 5;
  using Gm = Geo<D>;
  constexpr int ROWB = Gm::ROWB, TILEB = Gm::TILEB, NLD = Gm::NLD, KQ = Gm::KQ, MD = Gm::MD;
  typedef __attribute__((address_space(3))) void lds_void;
  __shared__ __attribute__((aligned(1024))) char lds_k0[TILEB];
  __shared__ __attribute__((aligned(1024))) char lds_v0[TILEB];
  __shared__ __attribute__((aligned(1024))) char lds_k1[TILEB];
  __shared__ __attribute__((aligned(1024))) char lds_v1[TILEB];
  // global modes: the positions of the global key tile held in each stage
  __shared__ __attribute__((aligned(16))) int lds_gp[2][kGlobal ? kBN : 1];

  // ---- which (query head, residue class, query block) this workgroup owns;
  // consecutive ids go round-robin to the 8 XCDs: each gets a contiguous range
  const int G = Hq / Hkv;
  int id = (int)blockIdx.x;
  const int nwg = (int)gridDim.x;
  if ((nwg & 7) == 0) id = (id & 7) * (nwg >> 3) + (id >> 3);
  const int hg = id % G;
  const int rest = id / G;
  const int qt = rest % n_qtiles;
  int kvh = rest / n_qtiles;
  const int cls = kvh % dil;
  kvh /= dil;
  const int h = kvh * G + hg;
  const int T = tm::class_rows(Tseq, cls, dil);  // rows of this residue class
  const int RS = dil * D;                        // floats between consecutive rows
  const int q0 = qt * kBM;
  if (q0 >= T) return;  // a shorter class: nothing to do (uniform over the workgroup)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int qw0 = q0 + wave * 32;
  const int qi = qw0 + (lane & 31);  // the query row this lane owns

  const float* qh = q + (size_t)h * Tseq * D + (size_t)cls * D;
  const float* kh = k + (size_t)kvh * Tseq * D + (size_t)cls * D;
  const float* vh = v + (size_t)kvh * Tseq * D + (size_t)cls * D;
  // global keys sit at sequence positions (outside any residue class)
  const float* kg = k + (size_t)kvh * Tseq * D;
  const float* vg = v + (size_t)kvh * Tseq * D;

  // chunk mode: position of the chunk's first token; the lowest key is -pstart
  int pstart = 0;
  if constexpr (kChunk) {
    pstart = pos[kvh / hkv_seq];
    if (pstart < 0) {  // inactive sequence: zero rows (uniform over the workgroup)
      if (qi < T) {
        float* orow = out + ((size_t)h * Tseq + qi) * D;
#pragma unroll
        for (int md = 0; md < Geo<D>::MD; ++md)
#pragma unroll
          for (int rq = 0; rq < 4; ++rq)
            *reinterpret_cast<float4*>(orow + 32 * md + 8 * rq + 4 * half) = make_float4(0.f, 0.f, 0.f, 0.f);
      }
      return;
    }
  }

  const int hw = W >> 1;
  const int lo = kCausal ? SWA_TM_CAUSAL_BLOCK_LO(q0, W, pstart) : SWA_TM_SYM_BLOCK_LO(q0, hw);
  const int hi = kCausal ? SWA_TM_CAUSAL_BLOCK_HI(q0, T) : SWA_TM_SYM_BLOCK_HI(q0, T, hw);
  const int kt0 = kChunk ? tm::floor_tile(lo) : lo / kBN;
  const int kt1 = hi / kBN;
  // global modes: the global key tiles follow the window's, as kt1+1 .. kt_end
  const int kt_end = kGlobal ? tm::global_tiles_end(kt1, ngl) : kt1;
  const bool wave_active = qw0 < T;
  const int qlast = SWA_TM_WAVE_LAST(qw0, T);
  const int wlo = SWA_TM_WAVE_LO(kCausal, qw0, W, hw, pstart);
  const int whi = SWA_TM_WAVE_HI(kCausal, qlast, T, hw);

  // ---- the lane's Q row as B operands: group j holds dims 8j + 4*half .. +3
  float4 qf[KQ];
#pragma unroll
  for (int j = 0; j < KQ; ++j) {
    qf[j] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (qi < T) qf[j] = *reinterpret_cast<const float4*>(qh + (size_t)qi * RS + 8 * j + 4 * half);
  }

  // ---- direct tile loads: load j of this thread fills the 16 bytes at LDS
  // offset (j * kThreads + tid) * 16 (each wave writes 1 KB contiguously) and
  // fetches the logical chunk the swizzle keeps there; rows past T re-read
  // row T - 1 (finite, masked)
  int src_row[NLD], src_koff[NLD];
#pragma unroll
  for (int j = 0; j < NLD; ++j) {
    const int o = tm::load_lds_offset(j, tid, kThreads);
    const int row = tm::load_row(o, ROWB);
    src_row[j] = row;
    src_koff[j] = (tm::load_chunk(o, ROWB) ^ swz<D>(row)) * 16;
  }
  auto load_tile = [&](char* Kdst, char* Vdst, int kt) __attribute__((always_inline)) {
    if constexpr (kGlobal) {
      if (kt > kt1) {
        // a global key tile: row j holds the key at gpos[t0 + j]; rows past
        // the last global key, and positions outside [0, Tseq), re-read a
        // valid row (masked); the tile's positions go to LDS for the mask
        // (written after the barrier that frees the stage)
        const int t0 = (kt - kt1 - 1) * kBN;
        if (tid < kBN) lds_gp[(kt - kt0) & 1][tid] = gpos[tm::global_index(t0, tid, ngl)];
        const __amdgpu_buffer_rsrc_t rk =
            __builtin_amdgcn_make_buffer_rsrc((void*)kg, 0, Tseq * ROWB, kBufferFlags);
        const __amdgpu_buffer_rsrc_t rv =
            __builtin_amdgcn_make_buffer_rsrc((void*)vg, 0, Tseq * ROWB, kBufferFlags);
#pragma unroll
        for (int j = 0; j < NLD; ++j) {
          const int wbase = (j * kThreads + wave * 64) * 16;
          const int roff = tm::global_src_row(gpos[tm::global_index(t0, src_row[j], ngl)], Tseq) * ROWB;
          const int koff = roff + src_koff[j];
          const int voff = roff + tm::load_chunk(tm::load_lds_offset(j, tid, kThreads), ROWB) * 16;
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass mishandles this builtin
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(Kdst + wbase), 16, koff, 0, 0, 0);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(Vdst + wbase), 16, voff, 0, 0, 0);
#else
          (void)rk, (void)rv, (void)wbase, (void)koff, (void)voff;
#endif
        }
        return;
      }
    }
    if constexpr (kChunk) {
      if (kt < 0) {
        // a ring tile: key r = kt * kBN + row is position pstart + r, in slot
        // (pstart + r) mod W; rows before position 0 (never in a window)
        // re-read position 0, which every sequence with pstart >= 1 has written
        const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(kring + (size_t)kvh * W * D), 0, W * ROWB, kBufferFlags);
        const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(vring + (size_t)kvh * W * D), 0, W * ROWB, kBufferFlags);
#pragma unroll
        for (int j = 0; j < NLD; ++j) {
          const int wbase = (j * kThreads + wave * 64) * 16;
          const int roff = (int)tm::ring_slot(pstart, kt * kBN, src_row[j], W) * ROWB;
          const int koff = roff + src_koff[j];
          const int voff = roff + tm::load_chunk(tm::load_lds_offset(j, tid, kThreads), ROWB) * 16;
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass mishandles this builtin
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(Kdst + wbase), 16, koff, 0, 0, 0);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(Vdst + wbase), 16, voff, 0, 0, 0);
#else
          (void)rk, (void)rv, (void)wbase, (void)koff, (void)voff;
#endif
        }
        return;
      }
    }
    const int last = tm::tile_last(T, kt);
    const int RSB = RS * 4;
    const int bytes = tm::tile_bytes(last, RSB, ROWB);
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc((void*)(kh + (size_t)kt * kBN * RS), 0, bytes, kBufferFlags);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc((void*)(vh + (size_t)kt * kBN * RS), 0, bytes, kBufferFlags);
#pragma unroll
    for (int j = 0; j < NLD; ++j) {
      const int wbase = (j * kThreads + wave * 64) * 16;
      const int roff = tm::tile_row_offset(src_row[j], last, RSB);
      const int koff = roff + src_koff[j];
      const int voff = roff + tm::load_chunk(tm::load_lds_offset(j, tid, kThreads), ROWB) * 16;
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass mishandles this builtin
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(Kdst + wbase), 16, koff, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(Vdst + wbase), 16, voff, 0, 0, 0);
#else
      (void)rk, (void)rv, (void)wbase, (void)koff, (void)voff;
#endif
    }
  };

  // per-lane LDS read offsets: K operand group j of LDS row l % 32 (+ the
  // block's first row; the swizzle repeats every 16 rows), V at row
  // 4 * half (+ the step's row) and dim l % 32 (+ 32 per output block)
  int koff[KQ];
#pragma unroll
  for (int j = 0; j < KQ; ++j) koff[j] = (lane & 31) * ROWB + (((2 * j + half) ^ swz<D>(lane & 31)) * 16);
  const int vbase = 4 * half * ROWB + (lane & 31) * 4;

  f32x16 o[MD];
#pragma unroll
  for (int md = 0; md < MD; ++md) o[md] = f32x16{};
  float m = -INFINITY;  // running maximum of the row's scaled scores (log2 units)
  float l = 0.f;        // this lane's share of the row sum

  // One 32-key block (keys k0 .. k0 + 31, LDS rows kb .. kb + 31 of the
  // tile): S^T, mask (blocks crossing a window edge or the sequence end; in a
  // global tile, gp holding the block's global positions and k0 the global
  // index of its first key: the keys that count for the row), online softmax,
  // O^T += V^T P^T.  The group barriers interleave each LDS
  // read with the products it feeds, one group ahead, so that the compiler
  // does not hoist every read of the block (and spill their registers).
  const int rpos = cls + dil * qi;  // this lane's row as a sequence position
  auto block = [&](const char* Ks, const char* Vs, int kb, int k0, bool full, const int* gp) __attribute__((always_inline)) {
    f32x16 sb = f32x16{};
#pragma unroll
    for (int j = 0; j < KQ; ++j) {
      const float4 kq = *reinterpret_cast<const float4*>(Ks + kb * ROWB + koff[j]);
      sb = __builtin_amdgcn_mfma_f32_32x32x2f32(kq.x, qf[j].x, sb, 0, 0, 0);
      sb = __builtin_amdgcn_mfma_f32_32x32x2f32(kq.y, qf[j].y, sb, 0, 0, 0);
      sb = __builtin_amdgcn_mfma_f32_32x32x2f32(kq.z, qf[j].z, sb, 0, 0, 0);
      sb = __builtin_amdgcn_mfma_f32_32x32x2f32(kq.w, qf[j].w, sb, 0, 0, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int j = 0; j < KQ; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      if (j + 2 < KQ) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);

    int gpv[16];
    if (kGlobal && gp) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int4 x = *reinterpret_cast<const int4*>(gp + 8 * g + 4 * half);
        gpv[4 * g] = x.x, gpv[4 * g + 1] = x.y, gpv[4 * g + 2] = x.z, gpv[4 * g + 3] = x.w;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float t = sb[r] * c;
      const int key = k0 + 8 * (r >> 2) + 4 * half + (r & 3);
      if (kGlobal && gp) {
        if (!tm::global_counts(kCausal, dil > 1, rpos, gpv[r], key, ngl, Tseq, W, dil)) t = -INFINITY;
      } else if (!full) {
        if (!tm::edge_visible(kCausal, qi, key, T, W, pstart)) t = -INFINITY;
      }
      sb[r] = t;
      mx = fmaxf(mx, t);
    }
    mx = max_lane_pair(mx);  // lanes l and l^32 hold the same row
    // The reference maximum m is raised only when the block's maximum exceeds
    // it by more than kGrow (or on the row's first keys), so that the
    // accumulators are rescaled rarely: probabilities up to 2^kGrow cost no
    // precision (fp32 is a relative-precision format) and the sums stay far
    // from overflow; the row's largest probability is at least 1, so nothing
    // that underflows against m would count next to it.
    const bool grow = mx > m + kGrow;  // m = -inf: any key of the row
    if (__ballot(grow)) {
      const float m_new = grow ? mx : m;
      const float alpha = __builtin_amdgcn_exp2f(m - (m_new == -INFINITY ? 0.f : m_new));
      m = m_new;
      l *= alpha;
#pragma unroll
      for (int md = 0; md < MD; ++md) {
#pragma unroll
        for (int r = 0; r < 16; ++r) o[md][r] *= alpha;
      }
    }
    const float m_use = m == -INFINITY ? 0.f : m;  // a row without keys so far
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      sb[r] = __builtin_amdgcn_exp2f(sb[r] - m_use);
      l += sb[r];
    }
    __builtin_amdgcn_sched_barrier(0);

#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      const int vrow = kb + 8 * (kk >> 2) + (kk & 3);  // + 4 * half, in vbase
#pragma unroll
      for (int md = 0; md < MD; ++md) {
        const float va = *reinterpret_cast<const float*>(Vs + vrow * ROWB + 128 * md + vbase);
        o[md] = __builtin_amdgcn_mfma_f32_32x32x2f32(va, sb[kk], o[md], 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * MD, 0);
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      __builtin_amdgcn_sched_group_barrier(0x008, MD, 0);
      if (kk + 2 < 16) __builtin_amdgcn_sched_group_barrier(0x100, MD, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // Wait for this tile's loads (issued during the previous one) and for every
  // wave to be done with the other stage, refill that stage, consume this one.
  auto step = [&](const char* Ks, const char* Vs, char* Kn, char* Vn, int kt) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    if (kt < kt_end) load_tile(Kn, Vn, kt + 1);
    const int k0 = kt * kBN;
    if (!tm::tile_visited(wave_active, wlo, whi, k0)) return;
    const bool full = tm::tile_full(kCausal, kChunk, k0, qw0, qlast, T, W, pstart);
    block(Ks, Vs, 0, k0, full, nullptr);
    block(Ks, Vs, 32, k0 + 32, full, nullptr);
  };
  load_tile(lds_k0, lds_v0, kt0);
  for (int kt = kt0; kt <= kt1; kt += 2) {
    step(lds_k0, lds_v0, lds_k1, lds_v1, kt);
    if (kt + 1 > kt1) break;
    step(lds_k1, lds_v1, lds_k0, lds_v0, kt + 1);
  }
  // global modes: the global key tiles (tile kt sits in stage (kt - kt0) & 1;
  // the last window step already requested the first of them); a 32-key
  // block without global keys is skipped
  if constexpr (kGlobal) {
    for (int kt = kt1 + 1; kt <= kt_end; ++kt) {
      const int st = (kt - kt0) & 1;
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      __syncthreads();
      if (kt < kt_end) load_tile(st ? lds_k0 : lds_k1, st ? lds_v0 : lds_v1, kt + 1);
      if (!wave_active) continue;
      const int t0 = (kt - kt1 - 1) * kBN;
      block(st ? lds_k1 : lds_k0, st ? lds_v1 : lds_v0, 0, t0, false, lds_gp[st]);
      if (ngl - t0 > 32) block(st ? lds_k1 : lds_k0, st ? lds_v1 : lds_v0, 32, t0 + 32, false, lds_gp[st] + 32);
    }
  }

  // ---- epilogue: divide by the row sum and store (the exchange involves
  // both wave halves, so it precedes the guard)
  const float l_tot = l + __shfl_xor(l, 32);
  if (qi < T) {
    const float inv = 1.0f / l_tot;
    float* orow = out + (size_t)h * Tseq * D + (size_t)cls * D + (size_t)qi * RS;
#pragma unroll
    for (int md = 0; md < MD; ++md) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        *reinterpret_cast<float4*>(orow + 32 * md + 8 * rq + 4 * half) =
            make_float4(o[md][4 * rq] * inv, o[md][4 * rq + 1] * inv, o[md][4 * rq + 2] * inv,
                        o[md][4 * rq + 3] * inv);
      }
    }
  }
}

template <int D, int MODE>
hipError_t launch(const void* q, const void* k, const void* v, void* out, int T, int W, int Hq,
                  int Hkv, float scale, int dil, hipStream_t stream,
                  const int32_t* gpos = nullptr, int ngl = 0) {
  // residue classes: the longest has ceil(T / dil) rows
  const int n_qtiles = ((T + dil - 1) / dil + f32m::kBM - 1) / f32m::kBM;
  const long long nwg = (long long)n_qtiles * Hq * dil;
  hipLaunchKernelGGL((prefill_f32_mfma_kernel<D, MODE>), dim3((unsigned)nwg),
                     dim3(f32m::kThreads), 0, stream, static_cast<const float*>(q),
                     static_cast<const float*>(k), static_cast<const float*>(v),
                     static_cast<float*>(out), T, W, Hq, Hkv, scale * kLog2e, n_qtiles, dil,
                     static_cast<const float*>(nullptr), static_cast<const float*>(nullptr),
                     static_cast<const int32_t*>(nullptr), 1, gpos, ngl);
  return hipGetLastError();
}

template <int D>
hipError_t launch_chunk(const void* q, const void* k, const void* v, const void* k_ring,
                        const void* v_ring, const int32_t* pos, void* out, int B, int n, int W,
                        int Hq, int Hkv, float scale, hipStream_t stream) {
  const int n_qtiles = (n + f32m::kBM - 1) / f32m::kBM;
  const long long nwg = (long long)n_qtiles * Hq * B;
  hipLaunchKernelGGL((prefill_f32_mfma_kernel<D, 2>), dim3((unsigned)nwg), dim3(f32m::kThreads), 0,
                     stream, static_cast<const float*>(q), static_cast<const float*>(k),
                     static_cast<const float*>(v), static_cast<float*>(out), n, W, Hq * B, Hkv * B,
                     scale * kLog2e, n_qtiles, 1, static_cast<const float*>(k_ring),
                     static_cast<const float*>(v_ring), pos, Hkv, static_cast<const int32_t*>(nullptr), 0);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_global_window_f32(const void* q, const void* k, const void* v,
                                            void* out, int T, int W, int Hq, int Hkv, int d,
                                            int mode, float scale, const int32_t* gpos, int ngl,
                                            int dil, hipStream_t stream) {
  if (mode == 0) {
    if (d == 32) return launch<32, 5>(q, k, v, out, T, W, Hq, Hkv, scale, dil, stream, gpos, ngl);
    if (d == 64) return launch<64, 5>(q, k, v, out, T, W, Hq, Hkv, scale, dil, stream, gpos, ngl);
    return launch<128, 5>(q, k, v, out, T, W, Hq, Hkv, scale, dil, stream, gpos, ngl);
  }
  if (d == 32) return launch<32, 6>(q, k, v, out, T, W, Hq, Hkv, scale, dil, stream, gpos, ngl);
  if (d == 64) return launch<64, 6>(q, k, v, out, T, W, Hq, Hkv, scale, dil, stream, gpos, ngl);
  return launch<128, 6>(q, k, v, out, T, W, Hq, Hkv, scale, dil, stream, gpos, ngl);
}

hipError_t launch_prefill_chunk_f32(const void* q, const void* k, const void* v,
                                    const void* k_ring, const void* v_ring, const int32_t* pos,
                                    void* out, int B, int n, int W, int Hq, int Hkv, int d,
                                    float scale, hipStream_t stream) {
  if (d == 32) return launch_chunk<32>(q, k, v, k_ring, v_ring, pos, out, B, n, W, Hq, Hkv, scale, stream);
  if (d == 64) return launch_chunk<64>(q, k, v, k_ring, v_ring, pos, out, B, n, W, Hq, Hkv, scale, stream);
  return launch_chunk<128>(q, k, v, k_ring, v_ring, pos, out, B, n, W, Hq, Hkv, scale, stream);
}

hipError_t launch_prefill_dilated_f32(const void* q, const void* k, const void* v, void* out,
                                      int T, int W, int Hq, int Hkv, int d, int mode, float scale,
                                      int dil, hipStream_t stream) {
  if (mode == 0) {
    if (d == 32) return launch<32, 0>(q, k, v, out, T, W, Hq, Hkv, scale, dil, stream);
    if (d == 64) return launch<64, 0>(q, k, v, out, T, W, Hq, Hkv, scale, dil, stream);
    return launch<128, 0>(q, k, v, out, T, W, Hq, Hkv, scale, dil, stream);
  }
  if (d == 32) return launch<32, 1>(q, k, v, out, T, W, Hq, Hkv, scale, dil, stream);
  if (d == 64) return launch<64, 1>(q, k, v, out, T, W, Hq, Hkv, scale, dil, stream);
  return launch<128, 1>(q, k, v, out, T, W, Hq, Hkv, scale, dil, stream);
}

hipError_t launch_prefill_f32(const void* q, const void* k, const void* v, void* out, int T,
                              int W, int Hq, int Hkv, int d, int mode, float scale,
                              hipStream_t stream) {
  return launch_prefill_dilated_f32(q, k, v, out, T, W, Hq, Hkv, d, mode, scale, 1, stream);
}

}  // namespace swa
