// Block-sparse ragged causal prefill on matrix cores.
//
// [FI] vllm.models.minimax_m3.nvidia.sparse_attention_flashinfer,
//      MiniMaxM3SparseFlashInferImpl.forward (msa_sparse_attention: ragged
//      rows by cu_seqlens_q, causal, per-token top-k blocks).
// [NV4] vllm.models.minimax_m3.amd.sparse_attention_nvfp4,
//      MiniMaxM3SparseRocmNvfp4Impl / MetadataBuilder.build (each prefill
//      token's request and absolute position).
// [SPA] vllm.models.minimax_m3.amd.ops.sparse_pa,
//      _write_sparse_block_table_row_from_values (the tokens a row sees).
//
// Work decomposition.  A workgroup (8 waves) owns one kv head and QT
// consecutive query rows of one request (QT = 32 for 8 query heads per kv
// head, 16 for 16).  Every query row picks its own blocks, so the workgroup
// first builds, per block of the request, the bit mask of its rows that
// selected it (and may see it causally), then walks the blocks some row
// selected in ascending order.  Each such block's K and V (128 keys x 256 B)
// go once into LDS by direct global-to-LDS loads (each lane's LDS slot is
// fixed, so layouts are made by choosing which global chunk a lane fetches):
// K double-buffered as [key][d] with 16-byte chunks XOR-swizzled by key, V
// as plain [key][d].  At each block boundary, while no copy is in flight, V
// is transposed LDS-to-LDS (8 keys x 8 d per thread, in registers) into V^T
// cells: for each 32-key chunk and d, the 8 keys of a lane group in the order
// the P operand holds them, placed so that both the transposing writes and
// the operand reads are free of bank conflicts.  Both operands are then plain
// 16-byte LDS reads, and the next block's copies overlap the compute.  Every
// wave
// owns 2 matrix tiles of 16 rows = (16 / G query rows) x (G heads) and runs
// QK^T and PV only for the tiles whose rows selected the block; the other
// rows of an active tile are masked.  Online softmax state stays in
// registers; the workgroup writes its rows' bf16 outputs at the end.
// Workgroups of one kv head share an XCD (blockIdx % Hkv), so K/V blocks
// re-read by neighbouring query tiles hit that XCD's L2.
#include "msa_device.h"
#include "msa_internal.h"

namespace msa {

constexpr int kPfWaves = 8;                 // two per SIMD: one's softmax overlaps the other's MFMAs
constexpr int kPfThreads = 64 * kPfWaves;
constexpr int kPfTiles = 2;                 // matrix tiles per wave
constexpr int kPfMaxBlocks = 2048;          // request blocks a workgroup can index
constexpr int kPfBlockBytes = kBlockTokens * 256;   // one block of K (or V), bf16, head_dim 128

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

// K row swizzle: 16-byte chunk c of key row k sits at chunk c ^ (k & 15).
__device__ __forceinline__ int k_swz(int key) { return key & 15; }

// V^T cell of (d, key group g) inside an 8 KB chunk: row (d/16, g) of 256 B,
// 16-byte cell (d % 16) ^ (d / 16).  Reads (16 lanes: d = 16 nn + r) and the
// transposing writes (16 lanes: d = 8 m + e) each touch 16 distinct cells of
// one 256-byte row or of distinct bank groups.
__device__ __forceinline__ int vt_cell(int d, int g) {
  return (((d >> 4) * 4 + g) << 8) + ((((d & 15) ^ (d >> 4)) & 15) << 4);
}

typedef __attribute__((address_space(3))) uint8_t lds_u8;

// K and V of block `phys` (logical block `blk`), kv head kvh, into LDS: 4 + 4
// direct 16-byte loads per lane.  Keys at or past seq_len are read from key 0
// of the block instead (finite data that gets probability zero), so no NaN
// of an unwritten slot reaches the products.
__device__ __forceinline__ void pf_issue_block(lds_u8* kb, lds_u8* vb, const AttendArgs& a, int kvh, int phys,
                                               int blk, int seq_len) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t pg = (int64_t)phys * a.block_page_stride;
  const int64_t head_off = (int64_t)kvh * kPageTokens * 256;
  const int nkeys = seq_len - blk * kBlockTokens;     // keys of this block that exist (>= 1)
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int P = (wave * 4 + s) * 1024 + lane * 16;  // LDS byte this lane fills
    const int key = P >> 8, pc = (P >> 4) & 15;
    const int src = key < nkeys ? key : 0;
    const int64_t row = (src >> 4) * a.page_stride + head_off + (src & 15) * 256;
    __builtin_amdgcn_global_load_lds(a.k_base + pg * a.page_stride + row + ((pc ^ k_swz(key)) << 4),
                                     kb + (wave * 4 + s) * 1024, 16, 0, 0);
    __builtin_amdgcn_global_load_lds(a.v_base + (pg + a.v_page_offset) * a.page_stride + row + (pc << 4),
                                     vb + (wave * 4 + s) * 1024, 16, 0, 0);
  }
}

// V [key][d] -> V^T cells.  Wave w handles 32-key chunk c = w / 2; lane
// (g, ml) of it takes keys tau(8g .. 8g+7) of the chunk (4g..4g+3 and
// 16+4g..16+4g+3) and d = 4m .. 4m+3 with m = 16 (w % 2) + ml.
__device__ __forceinline__ void pf_transpose_v(const uint8_t* vnat, uint8_t* vt) {
  const int tid = threadIdx.x, wave = tid >> 6, c = wave >> 1;
  const int g = (tid >> 4) & 3, m = 16 * (wave & 1) + (tid & 15);
  u32x2 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int key = c * 32 + (i < 4 ? 4 * g + i : 16 + 4 * g + (i - 4));
    v[i] = *reinterpret_cast<const u32x2*>(vnat + key * 256 + m * 8);
  }
  uint8_t* vc = vt + c * 8192;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    u32x4 o;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t a0 = v[2 * p][e >> 1], a1 = v[2 * p + 1][e >> 1];
      o[p] = (e & 1) ? pair_hi(a0, a1) : pair_lo(a0, a1);
    }
    *reinterpret_cast<u32x4*>(vc + vt_cell(4 * m + e, g)) = o;
  }
}

struct PfWave {
  static constexpr int KK = 4, NN = 8;
  bf16x8 qop[kPfTiles][KK];
  f32x4 acc[kPfTiles][NN];
  float m[kPfTiles], l[kPfTiles];
  int lrow[kPfTiles];     // row within the workgroup tile, or -1
  int lpos[kPfTiles];     // that row's absolute position
};

// Online softmax keeps, per (row, head), a reference max m and rescales the
// accumulators only when a chunk's max exceeds m by more than kLazy (log2
// units): probabilities are then at most 2^kLazy, well inside bf16 / fp32
// range, and the common case skips the rescale of 32 accumulators per tile.
constexpr float kLazy = 8.f;

// One selected block against this wave's tiles.  `causal` is set when the
// block can be the own block of a row of this workgroup (keys past a row's
// position must be masked); earlier blocks need only the row selection.
__device__ __forceinline__ void pf_compute_block(PfWave& w, const uint8_t* kb, const uint8_t* vtb, uint32_t bmask,
                                                 int blk, int wave, int RT, float sl2, bool causal) {
  constexpr int KK = PfWave::KK, NN = PfWave::NN;
  const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
  // per-lane LDS offsets (chunk / tile / step parts are compile-time)
  int koff[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) koff[kk] = r * 256 + (((4 * kk + g) ^ r) << 4);

  // per-tile row selection: bias 0 for a selected row, -inf otherwise
  float bias[kPfTiles];
  bool active[kPfTiles];
#pragma unroll
  for (int i = 0; i < kPfTiles; ++i) {
    const uint32_t tile_bits = ((1u << RT) - 1u) << ((wave * kPfTiles + i) * RT);
    active[i] = (bmask & tile_bits) != 0u;
    const bool sel = w.lrow[i] >= 0 && ((bmask >> w.lrow[i]) & 1u);
    bias[i] = sel ? 0.f : -INFINITY;
  }
  const int kpos_blk = blk * kBlockTokens;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    // operands of this 32-key chunk, shared by the wave's active tiles
    bf16x8 kop[2][KK];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        kop[tt][kk] = *reinterpret_cast<const bf16x8*>(kb + (c * 32 + 16 * tt) * 256 + koff[kk]);
    // V^T operand of output tile nn: lane (r, g) reads d = 16 nn + r, keys
    // tau(8g .. 8g+7) of the chunk: one 16-byte V^T cell.
    bf16x8 vop[NN];
#pragma unroll
    for (int nn = 0; nn < NN; ++nn)
      vop[nn] = *reinterpret_cast<const bf16x8*>(vtb + c * 8192 + vt_cell(16 * nn + r, g));
    const int kbase = kpos_blk + c * 32 + 4 * g;
#pragma unroll
    for (int i = 0; i < kPfTiles; ++i) {
      if (!active[i]) continue;
      f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        s0 = mfma16(kop[0][kk], w.qop[i][kk], s0);
        s1 = mfma16(kop[1][kk], w.qop[i][kk], s1);
      }
      float sv[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
      if (causal) {
#pragma unroll
        for (int ii = 0; ii < 8; ++ii) {
          const int kp = kbase + (ii & 3) + ((ii >> 2) << 4);
          sv[ii] = kp <= w.lpos[i] ? sv[ii] : -INFINITY;
        }
      }
      float mx = sv[0];
#pragma unroll
      for (int ii = 1; ii < 8; ++ii) mx = fmaxf(mx, sv[ii]);
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mxs = fmaf(mx, sl2, bias[i]);            // chunk max, scaled (log2 units)
      if (__ballot(mxs > w.m[i] + kLazy)) {                // rare after the first chunks
        const float m_new = fmaxf(w.m[i], mxs);
        const float alpha = exp2_fast(w.m[i] - (m_new == -INFINITY ? 0.f : m_new));
        w.l[i] *= alpha;
#pragma unroll
        for (int nn = 0; nn < NN; ++nn) w.acc[i][nn] = w.acc[i][nn] * alpha;
        w.m[i] = m_new;
      }
      const float off = bias[i] - (w.m[i] == -INFINITY ? 0.f : w.m[i]);
      float p[8], ps = 0.f;
#pragma unroll
      for (int ii = 0; ii < 8; ++ii) {
        p[ii] = exp2_fast(fmaf(sv[ii], sl2, off));
        ps += p[ii];
      }
      w.l[i] += ps;
      const u32x4 pw = {pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3]), pack_bf16(p[4], p[5]), pack_bf16(p[6], p[7])};
      const bf16x8 pop = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
      for (int nn = 0; nn < NN; ++nn) w.acc[i][nn] = mfma16(vop[nn], pop, w.acc[i][nn]);
    }
  }
}

__global__ __launch_bounds__(kPfThreads) void prefill_blocks_kernel(const AttendArgs a, int n_slots) {
  constexpr int D = 128, KK = PfWave::KK, NN = PfWave::NN;
  // two K/V buffers as distinct LDS objects: the loop below is unrolled by two,
  // so the compiler knows the in-flight copies target the other buffer
  __shared__ __align__(16) uint8_t k0[kPfBlockBytes], k1[kPfBlockBytes];
  __shared__ __align__(16) uint8_t vnat[kPfBlockBytes], vt[kPfBlockBytes];
  __shared__ uint32_t s_mask[kPfMaxBlocks];
  __shared__ uint16_t s_list[kPfMaxBlocks];   // selected blocks, ascending
  __shared__ int32_t s_phys[kPfMaxBlocks];    // their physical block ids
  __shared__ int s_info[4];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, g = lane >> 4;
  const int G = a.group, RT = 16 / G, QT = kPfWaves * kPfTiles * RT;
  const int kvh = blockIdx.x % a.num_kv_heads;
  const int t = n_slots - 1 - (int)(blockIdx.x / a.num_kv_heads);   // heavy (late) tiles first
  const int R = a.num_reqs;

  // ---- which rows: a tile of one request, padding rows, or nothing
  if (wave == 0) {
    int running = 0, found_req = -1, found_row0 = 0;
    for (int base = 0; base < R; base += 64) {
      const int rq = base + lane;
      const int n = rq < R ? (a.cu_seqlens_q[rq + 1] - a.cu_seqlens_q[rq] + QT - 1) / QT : 0;
      const int incl = wave_incl_scan(n, lane);
      const int excl = incl - n;
      const bool hit = rq < R && t >= running + excl && t < running + incl;
      const uint64_t hm = __ballot(hit);
      if (hm) {
        const int src = __ffsll((unsigned long long)hm) - 1;
        found_req = __shfl(rq, src);
        found_row0 = __shfl(rq < R ? a.cu_seqlens_q[rq] + (t - running - excl) * QT : 0, src);
      }
      running += __shfl(incl, 63);
    }
    if (lane == 0) {
      const int real_end = a.cu_seqlens_q[R];
      if (found_req >= 0) {
        s_info[0] = 0;
        s_info[1] = found_req;
        s_info[2] = found_row0;
        s_info[3] = min(found_row0 + QT, a.cu_seqlens_q[found_req + 1]);
      } else {
        const int p = t - running;   // padding tiles follow the real ones
        s_info[0] = 1;
        s_info[1] = 0;
        s_info[2] = real_end + p * QT;
        s_info[3] = min(real_end + (p + 1) * QT, a.total_rows);
      }
    }
  }
  __syncthreads();
  const int mode = s_info[0], req = s_info[1], row0 = s_info[2], row_end = s_info[3];
  if (row0 >= row_end) return;   // uniform: nothing to do
  if (mode == 1) {
    // padding rows attend nothing: zero their heads of this kv head
    const int per_row = G * D / 8;   // 16-byte stores
    for (int idx = tid; idx < (row_end - row0) * per_row; idx += kPfThreads) {
      const int rr = idx / per_row, wd = idx % per_row;
      uint8_t* dst = reinterpret_cast<uint8_t*>(a.out) +
                     (((int64_t)(row0 + rr) * a.num_q_heads + kvh * G) * D) * 2 + wd * 16;
      *reinterpret_cast<u32x4*>(dst) = u32x4{0u, 0u, 0u, 0u};
    }
    return;
  }
  const int cu0 = a.cu_seqlens_q[req], cu1 = a.cu_seqlens_q[req + 1];
  const int seq_len = a.seq_lens[req];
  const int ctx0 = seq_len - (cu1 - cu0);          // context before the new tokens
  const int pos_first = ctx0 + (row0 - cu0);
  const int pos_last = ctx0 + (row_end - 1 - cu0);
  const int nblk = pos_last < 0 ? 0 : min(pos_last / kBlockTokens + 1, a.bt_cols);
  const int32_t* bt_row = a.block_table + (int64_t)req * a.bt_stride;

  // ---- per-block masks of the rows that selected the block (and may see it)
  for (int j = tid; j < nblk; j += kPfThreads) s_mask[j] = 0u;
  __syncthreads();
  const int nrows = row_end - row0;
  for (int idx = tid; idx < nrows * a.topk_k; idx += kPfThreads) {
    const int rr = idx / a.topk_k, tk = idx - rr * a.topk_k;
    const int pos = pos_first + rr;
    const int blk = a.topk[(int64_t)(row0 + rr) * a.topk_stride + tk];
    if (pos >= 0 && blk >= 0 && blk <= pos / kBlockTokens && blk < nblk) atomicOr(&s_mask[blk], 1u << rr);
  }
  __syncthreads();
  // ---- selected blocks, ascending (blocks whose pages lie outside the cache are skipped)
  if (wave == 0) {
    int n = 0;
    for (int base = 0; base < nblk; base += 64) {
      const int j = base + lane;
      bool act = j < nblk && s_mask[j] != 0u;
      if (act) {
        const int phys = bt_row[j];
        const int64_t last = (int64_t)phys * a.block_page_stride + a.v_page_offset + kPagesPerBlock - 1;
        act = phys >= 0 && last < a.num_pages;
      }
      const uint64_t am = __ballot(act);
      const int rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(am >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)am, 0u));
      if (act) {
        s_list[n + rank] = (uint16_t)j;
        s_phys[n + rank] = bt_row[j];
      }
      n += __popcll(am);
    }
    if (lane == 0) s_info[0] = n;
  }

  // ---- this wave's query operands and row data
  PfWave w;
#pragma unroll
  for (int i = 0; i < kPfTiles; ++i) {
    const int rr = (wave * kPfTiles + i) * RT + r / G;
    const bool ok = r < RT * G && rr < nrows;
    w.lrow[i] = ok ? rr : -1;
    w.lpos[i] = pos_first + rr;
    w.m[i] = -INFINITY;
    w.l[i] = 0.f;
    const uint8_t* qrow = reinterpret_cast<const uint8_t*>(a.q) +
                          (((int64_t)(row0 + (ok ? rr : 0)) * a.num_q_heads + kvh * G + (r % G)) * D) * 2;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const u32x4 q4 = ok ? *reinterpret_cast<const u32x4*>(qrow + 2 * (32 * kk + 8 * g)) : u32x4{0u, 0u, 0u, 0u};
      w.qop[i][kk] = __builtin_bit_cast(bf16x8, q4);
    }
#pragma unroll
    for (int nn = 0; nn < NN; ++nn) w.acc[i][nn] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float kscale = a.k_scale ? *a.k_scale : 1.f;
  const float sl2 = a.softmax_scale * kscale * kLog2e;
  __syncthreads();
  const int n_act = s_info[0];

  if (n_act > 0) pf_issue_block((lds_u8*)k0, (lds_u8*)vnat, a, kvh, s_phys[0], s_list[0], seq_len);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const uint32_t wave_bits = ((1u << (kPfTiles * RT)) - 1u) << (wave * kPfTiles * RT);
  const int own_first = pos_first / kBlockTokens;   // blocks before it are wholly in every row's past
  for (int it = 0; it < n_act; it += 2) {
    // even step: K in k0; the next block's K goes to k1
    {
      pf_transpose_v(vnat, vt);
      __syncthreads();
      if (it + 1 < n_act) pf_issue_block((lds_u8*)k1, (lds_u8*)vnat, a, kvh, s_phys[it + 1], s_list[it + 1], seq_len);
      const int j = s_list[it];
      const uint32_t bmask = s_mask[j];
      if (bmask & wave_bits) pf_compute_block(w, k0, vt, bmask, j, wave, RT, sl2, j >= own_first);
      __builtin_amdgcn_s_waitcnt(0);   // this lane's copies of the next block have landed
      __syncthreads();
    }
    if (it + 1 >= n_act) break;
    // odd step: K in k1; the next block's K goes to k0
    {
      pf_transpose_v(vnat, vt);
      __syncthreads();
      if (it + 2 < n_act) pf_issue_block((lds_u8*)k0, (lds_u8*)vnat, a, kvh, s_phys[it + 2], s_list[it + 2], seq_len);
      const int j = s_list[it + 1];
      const uint32_t bmask = s_mask[j];
      if (bmask & wave_bits) pf_compute_block(w, k1, vt, bmask, j, wave, RT, sl2, j >= own_first);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  }

  // ---- outputs: lane holds head r % G of row lrow, d = 16 nn + 4 g + ii
  const float vscale = a.v_scale ? *a.v_scale : 1.f;
#pragma unroll
  for (int i = 0; i < kPfTiles; ++i) {
    float L = w.l[i];
    L += __shfl_xor(L, 16);
    L += __shfl_xor(L, 32);
    if (w.lrow[i] < 0) continue;
    const float inv = L > 0.f ? vscale / L : 0.f;
    uint8_t* orow = reinterpret_cast<uint8_t*>(a.out) +
                    (((int64_t)(row0 + w.lrow[i]) * a.num_q_heads + kvh * G + (r % G)) * D) * 2;
#pragma unroll
    for (int nn = 0; nn < NN; ++nn) {
      const int d = 16 * nn + 4 * g;
      const u32x2 o = {pack_bf16(w.acc[i][nn][0] * inv, w.acc[i][nn][1] * inv),
                       pack_bf16(w.acc[i][nn][2] * inv, w.acc[i][nn][3] * inv)};
      *reinterpret_cast<u32x2*>(orow + d * 2) = o;
    }
  }
}

hipError_t launch_prefill_blocks(const AttendArgs& a, hipStream_t stream) {
  const int QT = kPfWaves * kPfTiles * (16 / a.group);
  const int n_slots = (a.total_rows + QT - 1) / QT + a.num_reqs + 1;
  const int64_t blocks = (int64_t)n_slots * a.num_kv_heads;
  hipLaunchKernelGGL(prefill_blocks_kernel, dim3((unsigned)blocks), dim3(kPfThreads), 0, stream, a, n_slots);
  return hipGetLastError();
}

bool prefill_blocks_supported(int group, int head_dim, int fmt, int bt_cols) {
  return (group == 8 || group == 16) && head_dim == 128 && fmt == kFmtBf16 && bt_cols <= kPfMaxBlocks;
}

}  // namespace msa
