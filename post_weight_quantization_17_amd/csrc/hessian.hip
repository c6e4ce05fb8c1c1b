// Stage 1 of the GPTQ layer path: H (+)= 2 X^T X.
//
// aiqz.cc "GPTQ：一键量化大模型压缩", section 二阶信息: the Hessian of the layer
// objective is twice the sum over calibration inputs of x x^T. X arrives as
// tokens x channels, so H = 2 X^T X: a symmetric rank-N update whose
// reduction runs over tokens.
//
// Design (gfx950):
//  * Only upper 256x256 tiles (bi <= bj) are computed. Each workgroup
//    (4 waves, 2x2, each wave 128x128 = 4x4 MFMA 32x32x16 f16 tiles) owns one
//    tile for one contiguous token range (split-K).
//  * X is copied from HBM straight into LDS (global_load_lds, 16 bytes per
//    lane) in its natural token-major layout, in four stages of 32 tokens:
//    the loads of step k+3 are in flight while step k's MFMAs run; no
//    registers or VALU work are spent on staging. MFMA operands need 8
//    consecutive tokens of one channel per lane: they are read with the
//    gfx950 transposing LDS read
//    (ds_read_b64_tr_b16), two per fragment, at per-lane base + immediate
//    offsets. Ragged tokens or channels take a checked register path into
//    the same layout.
//  * fp16 products are exact in fp32 and MFMA accumulates in fp32. Each
//    split writes its partial tile to the workspace; a second kernel sums the
//    splits in a fixed order in fp64, scales by 2, mirrors the upper tiles
//    into both triangles and applies accumulate. No atomics: deterministic.
//  * fp32 inputs take the fp32 MFMA (v_mfma_f32_32x32x2f32) on 64x64 tiles
//    with the same token splits, partials and reduction; X is not rounded
//    to fp16.
#include "gptq_common.h"

namespace gptq {
namespace {

constexpr int SY_T = 256;         // tile edge (fp16 MFMA kernel)
constexpr int SY_BK = 32;         // tokens per LDS stage
constexpr int SY_THREADS = 256;
constexpr int SYF_T = 64;         // tile edge (fp32 MFMA kernel)
constexpr int SYF_BK = 16;

// Upper-triangle tile index -> (bi, bj), row-major over bi <= bj.
__device__ __forceinline__ void tile_coords(int tile, int nb, int& bi, int& bj) {
  int r = 0, t = tile;
  while (t >= nb - r) {
    t -= nb - r;
    ++r;
  }
  bi = r;
  bj = r + t;
}

__host__ __device__ __forceinline__ int tile_index(int bi, int bj, int nb) {
  return bi * nb - (bi * (bi - 1)) / 2 + (bj - bi);
}

// LDS byte offset of the 16-byte chunk holding tokens [8 to, 8 to + 8) of
// channel ch inside one [256 channel][32 token] fp16 panel. The row
// permutation and chunk XOR keep both the transposing writes (channels
// 8c+v, c varying) and the MFMA fragment reads (32 consecutive channels)
// spread over distinct banks.
__device__ __forceinline__ int panel_off(int ch, int to) {
  const int row = ch ^ ((ch >> 3) & 3);
  const int chunk = to ^ ((ch >> 2) & 3) ^ ((ch >> 5) & 3);
  return row * 64 + chunk * 16;
}

__device__ __forceinline__ uint32_t lo_pair(uint32_t a, uint32_t b) {  // (a.lo, b.lo)
  return (a & 0xffffu) | (b << 16);
}
__device__ __forceinline__ uint32_t hi_pair(uint32_t a, uint32_t b) {  // (a.hi, b.hi)
  return (a >> 16) | (b & 0xffff0000u);
}

// Checked path: for every split either the edge tiles (bi, nb - 1) when d is
// not a multiple of 256 (all_tiles = 0) or every tile (all_tiles = 1, used
// when rows are not 16-byte aligned), plus the token tail (n_tokens % 32) of
// every tile into the extra slot `nsplit`.
// Tiles are read with bounds-checked 16-byte loads, transposed in registers
// and stored in a swizzled [channel][token] LDS layout.
__global__ void __launch_bounds__(SY_THREADS, 1)
syrk_f16_generic(const __half* __restrict__ X, int64_t n_tokens, int64_t n_full, int d, int64_t ldx, int nb,
                 int ntiles, int64_t tokens_per_split, int nsplit, int n_edge, int all_tiles,
                 float* __restrict__ partial) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[2][2][SY_T * SY_BK * 2];

  int tile, slot, bi, bj;
  int64_t kbeg, kend;
  if (int(blockIdx.x) < n_edge * nsplit) {
    const int e = blockIdx.x % n_edge;
    slot = blockIdx.x / n_edge;
    if (all_tiles) {
      tile = e;
      tile_coords(tile, nb, bi, bj);
    } else {
      bi = e;
      bj = nb - 1;
      tile = tile_index(bi, bj, nb);
    }
    kbeg = int64_t(slot) * tokens_per_split;
    kend = kbeg + tokens_per_split < n_full ? kbeg + tokens_per_split : n_full;
  } else {
    tile = blockIdx.x - n_edge * nsplit;
    tile_coords(tile, nb, bi, bj);
    slot = nsplit;
    kbeg = n_full;
    kend = n_tokens;
  }
  const bool diag = (bi == bj);
  const int I0 = bi * SY_T, J0 = bj * SY_T;
  const int nsteps = kend > kbeg ? int((kend - kbeg + SY_BK - 1) / SY_BK) : 0;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // Loader role: panel p, channel octet c, token octet to.
  const int lp = tid >> 7;
  const int lu = tid & 127;
  const int lc = lu & 31;
  const int lto = lu >> 5;
  const bool loader = !(diag && lp == 1);
  const int lch0 = (lp == 0 ? I0 : J0) + 8 * lc;
  const bool vec_ok = (lch0 + 8 <= d) && ((ldx & 7) == 0) &&
                      ((reinterpret_cast<uintptr_t>(X) & 15) == 0);

  uint4 in[8];
  auto gload = [&](int step) {
    const int64_t t0 = kbeg + int64_t(step) * SY_BK + 8 * lto;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int64_t t = t0 + r;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (loader && t < kend) {
        const __half* p = X + t * ldx + lch0;
        if (vec_ok) {
          v = *reinterpret_cast<const uint4*>(p);
        } else {
          unsigned short h[8];
#pragma unroll
          for (int e = 0; e < 8; ++e)
            h[e] = (lch0 + e < d) ? __half_as_ushort(p[e]) : (unsigned short)0;
          v.x = h[0] | (uint32_t(h[1]) << 16);
          v.y = h[2] | (uint32_t(h[3]) << 16);
          v.z = h[4] | (uint32_t(h[5]) << 16);
          v.w = h[6] | (uint32_t(h[7]) << 16);
        }
      }
      in[r] = v;
    }
  };
  auto lstore = [&](int stage) {
    if (!loader) return;
    unsigned char* base = lds[stage][lp];
    const uint32_t* w = reinterpret_cast<const uint32_t*>(in);
    // in[r] word h = channels (2h, 2h+1) of token r.
#pragma unroll
    for (int h = 0; h < 4; ++h) {
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        uint4 o;
        uint32_t* ow = reinterpret_cast<uint32_t*>(&o);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const uint32_t a = w[(2 * m) * 4 + h], c = w[(2 * m + 1) * 4 + h];
          ow[m] = b ? hi_pair(a, c) : lo_pair(a, c);
        }
        const int ch = 8 * lc + 2 * h + b;
        *reinterpret_cast<uint4*>(base + panel_off(ch, lto)) = o;
      }
    }
  };

  floatx16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx16{0};

  if (nsteps > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();
  for (int s = 0; s < nsteps; ++s) {
    const int st = s & 1;
    if (s + 1 < nsteps) gload(s + 1);
    const unsigned char* pa = lds[st][0];
    const unsigned char* pb = diag ? lds[st][0] : lds[st][1];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int to = 2 * kk + (lane >> 5);
      half8 a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ch = wm * 128 + i * 32 + (lane & 31);
        a[i] = *reinterpret_cast<const half8*>(pa + panel_off(ch, to));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int ch = wn * 128 + j * 32 + (lane & 31);
        b[j] = *reinterpret_cast<const half8*>(pb + panel_off(ch, to));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (s + 1 < nsteps) lstore(st ^ 1);
    __syncthreads();
  }

  // Partial tile, row-major [256][256]. 32x32 MFMA result layout: lane l holds
  // column l%32 and rows 8*(r/4) + 4*(l/32) + r%4 for register r.
  float* out = partial + (int64_t(slot) * ntiles + tile) * (SY_T * SY_T);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * 128 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int col = wn * 128 + j * 32 + (lane & 31);
        out[row * SY_T + col] = acc[i][j][r];
      }
}

// LDS layout of one panel stage: 32 tokens x 256 fp16 channels, token-major
// (each token row is its 512 contiguous bytes). Token t sits in slot
// (t % 16) at half (t / 16): byte (t % 16) * PITCH + (t / 16) * 512. The
// 64-byte pad per slot pair puts 4 consecutive tokens on 4 distinct 64-byte
// bank groups, so transposing reads of a 4-token x 16-channel block are
// conflict free, and one 1 KB direct-to-LDS load instruction (64 lanes x
// 16 bytes) fills exactly one slot pair (tokens t and t + 16).
constexpr int S_PITCH = 1088;
constexpr int S_PANEL = 16 * S_PITCH;  // 17408 bytes
constexpr int S_STAGE = 2 * S_PANEL;

typedef short short4v __attribute__((ext_vector_type(4)));
typedef short short8v __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) short4v lds_short4;

__device__ __forceinline__ half8 tr_frag(const unsigned char* lds, int off) {
  // Two transposing reads: lanes 4r..4r+3 of each 16-lane group fetch token
  // r of a 4-token x 16-channel block; lane i receives channel i's 4 tokens.
  const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(lds + off));
  const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(lds + off + 4 * S_PITCH));
  const short8v v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(half8, v);
}

// Interior tiles (both panels inside the matrix), whole 128-token blocks of
// 4 steps. Four LDS stages: stage s + 3 is loaded while stage s is computed;
// the schedule of one step is described at its definition below.
constexpr int S_NSTAGE = 4;

// Work order (XCD aware). Workgroups are dispatched round-robin over the 8
// XCDs (blockIdx % 8), each with its own L2. The host lists the interior
// tiles in 4x4 super-block order and cuts the list into 8 equal contiguous
// chunks, chunk x for XCD x: blockIdx = 8 (split * per + t) + x runs tile
// chunk_x[t] of `split`. All XCDs then stream the same token split at the
// same time (shared through the last-level cache) while each XCD's tiles
// cover few panels (reused in its L2).
constexpr int S_MAXMAP = 1800;
struct TileMap {
  int per;                     // tiles per XCD chunk (padded with -1)
  unsigned short t[S_MAXMAP];  // [8][per] global tile indices (0xffff = none)
};

__global__ void __launch_bounds__(SY_THREADS, 1)
syrk_f16_lds(const __half* __restrict__ X, int64_t n_main, int64_t ldx, int nb, int nbf, int n_int,
             int64_t tokens_per_split, int nsplit, float* __restrict__ partial, TileMap map) {
  // Separate objects per stage, so the compiler can see that the loads into
  // one stage never alias the reads of another.
  __shared__ __attribute__((aligned(16))) unsigned char lds0[S_STAGE];
  __shared__ __attribute__((aligned(16))) unsigned char lds1[S_STAGE];
  __shared__ __attribute__((aligned(16))) unsigned char lds2[S_STAGE];
  __shared__ __attribute__((aligned(16))) unsigned char lds3[S_STAGE];

  int tile, split, bi, bj;
  if (map.per > 0) {
    const int x = blockIdx.x & 7, k = blockIdx.x >> 3;
    split = k / map.per;
    const int tt = map.t[x * map.per + k % map.per];
    if (tt == 0xffff || split >= nsplit) return;  // padding slot
    tile = tt;
    tile_coords(tile, nb, bi, bj);
  } else {
    const int it = blockIdx.x % n_int;
    split = blockIdx.x / n_int;
    tile_coords(it, nbf, bi, bj);
    tile = tile_index(bi, bj, nb);
  }
  const int ntiles = nb * (nb + 1) / 2;
  const int I0 = bi * SY_T, J0 = bj * SY_T;
  const int64_t kbeg = int64_t(split) * tokens_per_split;
  const int64_t kend = kbeg + tokens_per_split < n_main ? kbeg + tokens_per_split : n_main;
  const int nsteps = int((kend - kbeg) / SY_BK);  // a multiple of S_NSTAGE

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // Each wave issues 8 direct loads per stage: slot pairs wave + 4u of panel
  // A (u < 4) and of panel B (u >= 4). A load fills one slot pair: lanes
  // 0-31 token (pair), lanes 32-63 token (pair + 16), 8 channels per lane.
  // Per-lane 32-bit element offsets from a per-step uniform base.
  uint32_t voff[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int pair = wave + 4 * (u & 3);
    const int P0 = u < 4 ? I0 : J0;
    voff[u] = uint32_t((pair + 16 * (lane >> 5)) * ldx + P0 + 8 * (lane & 31));
  }
  auto issue = [&](int step, unsigned char* buf) {
    const __half* xs = X + (kbeg + int64_t(step) * SY_BK) * ldx;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int pair = wave + 4 * (u & 3);
      unsigned char* l = buf + (u >> 2) * S_PANEL + pair * S_PITCH;
      __builtin_amdgcn_global_load_lds(xs + voff[u], (__attribute__((address_space(3))) void*)l, 16, 0, 0);
    }
  };

  // Per-lane base of the transposing fragment reads: 16-lane group g covers
  // 16 channels (16 * (g & 1) ..) for tokens 8 * (g >> 1) + [0, 4); within
  // the group lane 4r + q reads token r, channels 4q .. 4q + 3.
  const int g = lane >> 4, r = (lane >> 2) & 3, q = lane & 3;
  const int lane_off = (8 * (g >> 1) + r) * S_PITCH + 2 * (16 * (g & 1) + 4 * q);
  const int a_base = lane_off + 2 * (wm * 128);
  const int b_base = S_PANEL + lane_off + 2 * (wn * 128);

  floatx16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx16{0};

  half8 fa0[4], fb0[4], fa1[4], fb1[4];  // fragments: first / last 16 tokens
  auto read_frags = [&](const unsigned char* base, int kk, half8* fa, half8* fb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[i] = tr_frag(base, a_base + 64 * i + 512 * kk);
#pragma unroll
    for (int j = 0; j < 4; ++j) fb[j] = tr_frag(base, b_base + 64 * j + 512 * kk);
  };
  auto mfma16 = [&](const half8* fa, const half8* fb) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[i], fb[j], acc[i][j], 0, 0, 0);
  };
  // One step s (32 tokens) in two MFMA groups of 16, with the LDS reads and
  // the direct loads placed between the MFMAs (one wave per SIMD, so a read
  // issued after a group would leave the matrix pipe idle while it lands):
  //   group A: MFMAs on stage s, tokens 0-15 (fa0/fb0), interleaved with the
  //            loads of stage s + 3 and the reads of stage s, tokens 16-31
  //   wait:    own loads of stage s + 1 landed (stages s + 2 and s + 3 stay in
  //            flight: vmcnt 16), own LDS reads done; barrier
  //   group B: MFMAs on stage s, tokens 16-31 (fa1/fb1), interleaved with the
  //            reads of stage s + 1, tokens 0-15
  // The barrier of step s orders every hand-off: stage s + 1 has landed for
  // all waves before group B reads it, and every wave has finished reading
  // stage s - 1 (groups A and B of earlier steps) before group A of step s
  // loads stage s + 3 into that buffer. Loads past the last step re-load the
  // last step (valid memory, never read), so the load count per step, and
  // with it the vmcnt of the wait, is constant.
  auto step = [&](int s, unsigned char* cur, unsigned char* next, unsigned char* later) {
    issue(s + 3 < nsteps ? s + 3 : nsteps - 1, later);
    read_frags(cur, 1, fa1, fb1);
    mfma16(fa0, fb0);
    // Reads and loads go with the first 8 MFMAs, so they land while the
    // last 8 run.
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS reads
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // direct load
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0x4070);  // vmcnt(16) expcnt(7) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    read_frags(next, 0, fa0, fb0);
    mfma16(fa1, fb1);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    __builtin_amdgcn_sched_barrier(0);
  };

  if (nsteps > 0) {
    issue(0, lds0);
    issue(1 < nsteps ? 1 : nsteps - 1, lds1);
    issue(2 < nsteps ? 2 : nsteps - 1, lds2);
    __builtin_amdgcn_s_waitcnt(0x4070);  // stage 0 landed (vmcnt 16)
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    read_frags(lds0, 0, fa0, fb0);
  }
  for (int s = 0; s < nsteps; s += S_NSTAGE) {
    step(s, lds0, lds1, lds3);
    step(s + 1, lds1, lds2, lds0);
    step(s + 2, lds2, lds3, lds1);
    step(s + 3, lds3, lds0, lds2);
  }
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0): no direct load outlives the workgroup's LDS

  // Partial tile, row-major [256][256]. 32x32 MFMA result layout: lane l holds
  // column l%32 and rows 8*(r/4) + 4*(l/32) + r%4 for register r.
  float* out = partial + (int64_t(split) * ntiles + tile) * (SY_T * SY_T);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int row = wm * 128 + i * 32 + 8 * (rr >> 2) + 4 * (lane >> 5) + (rr & 3);
        const int col = wn * 128 + j * 32 + (lane & 31);
        out[row * SY_T + col] = acc[i][j][rr];
      }
}

// fp32 inputs: the same upper 64x64 tiles and token splits, on the fp32
// MFMA. Four waves (2x2) each own a 32x32 block: one v_mfma_f32_32x32x2f32
// per 2 tokens, whose A operand (lane l: channel I0 + 32 wi + l % 32, token
// l / 32) and B operand (channel J0 + 32 wj + l % 32, same token) are
// consecutive floats of one token row of the token-major LDS panels, so the
// 64 lanes read without bank conflicts. The products and sums are fp32, as
// the inputs are (no rounding of X to a narrower type).
__global__ void __launch_bounds__(256)
syrk_f32_mfma(const float* __restrict__ X, int64_t n_tokens, int d, int64_t ldx, int nb, int ntiles,
              int64_t tokens_per_split, float* __restrict__ partial) {
  __shared__ float sa[SYF_BK][SYF_T];
  __shared__ float sb[SYF_BK][SYF_T];
  const int tile = blockIdx.x % ntiles;
  const int split = blockIdx.x / ntiles;
  int bi, bj;
  tile_coords(tile, nb, bi, bj);
  const int I0 = bi * SYF_T, J0 = bj * SYF_T;
  const int64_t kbeg = int64_t(split) * tokens_per_split;
  int64_t kend = kbeg + tokens_per_split;
  if (kend > n_tokens) kend = n_tokens;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wi = wave >> 1, wj = wave & 1;
  const int lk = lane >> 5, lc = lane & 31;
  floatx16 acc = floatx16{0};
  for (int64_t k0 = kbeg; k0 < kend; k0 += SYF_BK) {
    for (int e = tid; e < SYF_BK * SYF_T; e += 256) {
      const int kk = e / SYF_T, c = e % SYF_T;
      const int64_t t = k0 + kk;
      sa[kk][c] = (t < kend && I0 + c < d) ? X[t * ldx + I0 + c] : 0.f;
      sb[kk][c] = (t < kend && J0 + c < d) ? X[t * ldx + J0 + c] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < SYF_BK; kk += 2) {
      const float a = sa[kk + lk][32 * wi + lc];
      const float b = sb[kk + lk][32 * wj + lc];
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
    }
    __syncthreads();
  }
  // 32x32 result layout: lane l holds column l % 32 and rows
  // 8 (r / 4) + 4 (l / 32) + r % 4 of register r.
  float* out = partial + (int64_t(split) * ntiles + tile) * (SYF_T * SYF_T);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = 32 * wi + 8 * (r >> 2) + 4 * lk + (r & 3);
    out[row * SYF_T + 32 * wj + lc] = acc[r];
  }
}

// H[i][j] = 2 * sum_s partial_s (min(i,j), max(i,j)) (+ H[i][j] if accumulate).
// One 32x32 source block (SI <= SJ, upper) per workgroup: its partials are
// read once and summed in a fixed split order in fp64, then the block is
// written to (SI, SJ) and, transposed through LDS, to (SJ, SI). A block on
// the diagonal mirrors its upper half.
__global__ void __launch_bounds__(256)
syrk_reduce(const float* __restrict__ partial, int T, int nb, int ntiles, int nsplit, int d,
            float* __restrict__ H, int accumulate) {
  __shared__ double blk[32][33];
  const int nob = (d + 31) / 32;
  int b = int(blockIdx.x), SI = 0;
  while (b >= nob - SI) {  // row SI of the upper triangle holds nob - SI blocks
    b -= nob - SI;
    ++SI;
  }
  const int SJ = SI + b;
  const int R0 = SI * 32, C0 = SJ * 32;
  const int bi = R0 / T, bj = C0 / T;
  const int tile = bi * nb - (bi * (bi - 1)) / 2 + (bj - bi);
  const int tid = threadIdx.x;
  for (int e = tid; e < 32 * 32; e += 256) {
    const int r = e >> 5, c = e & 31;
    const int gr = R0 + r, gc = C0 + c;
    double s = 0.0;
    if (gr < d && gc < d) {
      // Fixed order: splits 0, 1, 2, ... (loads batched 8 at a time).
      const int64_t off = int64_t(tile) * T * T + int64_t(gr - bi * T) * T + (gc - bj * T);
      const int64_t stride = int64_t(ntiles) * T * T;
      int sp = 0;
      for (; sp + 8 <= nsplit; sp += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = partial[(sp + u) * stride + off];
#pragma unroll
        for (int u = 0; u < 8; ++u) s += double(v[u]);
      }
      for (; sp < nsplit; ++sp) s += double(partial[sp * stride + off]);
    }
    blk[r][c] = s;
  }
  __syncthreads();
  for (int e = tid; e < 32 * 32; e += 256) {
    const int r = e >> 5, c = e & 31;
    {
      const int gi = R0 + r, gj = C0 + c;
      if (gi < d && gj < d) {
        double v = SI < SJ ? blk[r][c] : (r <= c ? blk[r][c] : blk[c][r]);
        v *= 2.0;
        const int64_t o = int64_t(gi) * d + gj;
        if (accumulate) v += double(H[o]);
        H[o] = float(v);
      }
    }
    if (SI < SJ) {
      const int gi = C0 + r, gj = R0 + c;
      if (gi < d && gj < d) {
        double v = blk[c][r] * 2.0;
        const int64_t o = int64_t(gi) * d + gj;
        if (accumulate) v += double(H[o]);
        H[o] = float(v);
      }
    }
  }
}

__global__ void fill_zero_f32(float* p, int64_t n) {
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < n; i += int64_t(gridDim.x) * blockDim.x)
    p[i] = 0.f;
}

struct SyrkPlan {
  int T, nb, ntiles, nsplit, nslot;
  int nbf, n_int, n_edge;  // fp16: interior blocks/tiles, edge tiles
  int64_t tokens_per_split, n_full;
  size_t ws_bytes;
};

// Token splits over the whole 32-token steps ([0, n_full)): enough
// workgroups to keep 256 CUs busy for several rounds and at least 4 partial
// sums per tile. fp16 inputs put the token tail (n_tokens % 32) of every
// tile in one extra slot; fp32 inputs split all tokens.
SyrkPlan plan_syrk(int64_t n_tokens, int64_t d, int xdtype) {
  SyrkPlan p{};
  const bool f16 = xdtype == GPTQ_F16;
  const int bk = f16 ? SY_BK : SYF_BK;
  p.T = f16 ? SY_T : SYF_T;
  p.nb = int((d + p.T - 1) / p.T);
  p.ntiles = p.nb * (p.nb + 1) / 2;
  // fp16: splits cover whole blocks of 4 steps (128 tokens), the rest of the
  // tokens is the tail.
  const int unit = f16 ? bk * S_NSTAGE : bk;
  p.n_full = f16 ? (n_tokens / unit) * unit : n_tokens;
  const int64_t ksteps = (p.n_full + unit - 1) / unit;
  int64_t want = (2048 + p.ntiles - 1) / p.ntiles;
  if (want < 4) want = 4;
  if (f16) {
    // One workgroup per CU at a time: among 4 .. 2 want splits, take the
    // count whose last round of 256 workgroups is fullest (ties: fewer
    // splits, i.e. fewer partial tiles to reduce).
    const int64_t tiles = int64_t(d / p.T) * (d / p.T + 1) / 2;
    if (tiles > 0) {
      double best = -1.0;
      int64_t pick = want;
      for (int64_t n = 4; n <= 2 * want; ++n) {
        const double rounds = double(tiles * n) / 256.0;
        const double eff = rounds / double(int64_t(rounds) + (rounds > double(int64_t(rounds)) ? 1 : 0));
        if (eff > best + 0.005) {
          best = eff;
          pick = n;
        }
      }
      want = pick;
    }
  }
  if (want > ksteps) want = ksteps;
  if (want < 1) want = 1;
  p.tokens_per_split = ((ksteps + want - 1) / want) * unit;
  p.nsplit = p.n_full > 0 ? int((p.n_full + p.tokens_per_split - 1) / p.tokens_per_split) : 0;
  p.nslot = p.nsplit + ((f16 && n_tokens > p.n_full) ? 1 : 0);
  p.nbf = f16 ? int(d / p.T) : 0;
  p.n_int = p.nbf * (p.nbf + 1) / 2;
  p.n_edge = (f16 && d % p.T != 0) ? p.nb : 0;
  p.ws_bytes = align_up(size_t(p.nslot) * p.ntiles * p.T * p.T * sizeof(float), 256);
  return p;
}

}  // namespace
}  // namespace gptq

using namespace gptq;

extern "C" size_t gptq_hessian_workspace_size(int64_t n_tokens, int64_t d, int xdtype) {
  if (d < 1 || n_tokens < 0 || (xdtype != GPTQ_F16 && xdtype != GPTQ_F32)) return 0;
  return plan_syrk(n_tokens, d, xdtype).ws_bytes;
}

extern "C" int gptq_hessian_accumulate(const void* X, int xdtype, int64_t n_tokens, int64_t d, int64_t ldx,
                                       float* H, int accumulate, void* ws, size_t ws_bytes, void* stream) {
  if (d < 1 || d > (1 << 20) || n_tokens < 0 || ldx < d || H == nullptr) return GPTQ_E_INVALID_ARG;
  if (xdtype != GPTQ_F16 && xdtype != GPTQ_F32) return GPTQ_E_INVALID_ARG;
  if (n_tokens > 0 && X == nullptr) return GPTQ_E_INVALID_ARG;
  hipStream_t s = as_stream(stream);
  if (n_tokens == 0) {
    if (!accumulate) {
      hipLaunchKernelGGL(fill_zero_f32, dim3(1024), dim3(256), 0, s, H, d * d);
      return launch_status();
    }
    return GPTQ_OK;
  }
  const SyrkPlan p = plan_syrk(n_tokens, d, xdtype);
  if (ws == nullptr || ws_bytes < p.ws_bytes) return GPTQ_E_WORKSPACE;
  float* partial = static_cast<float*>(ws);
  if (xdtype == GPTQ_F16) {
    const __half* Xh = static_cast<const __half*>(X);
    // Direct-to-LDS loads need 16-byte aligned rows.
    // (and per-lane offsets below 32 tokens x ldx must fit in 32 bits).
    const bool direct = ((ldx & 7) == 0) && ((reinterpret_cast<uintptr_t>(X) & 15) == 0) && ldx < (int64_t(1) << 26);
    int n_edge = p.n_edge, nbf = p.nbf, n_int = p.n_int;
    if (!direct) {  // every tile takes the checked path
      n_edge = 0;
      nbf = 0;
      n_int = 0;
    }
    if (n_int > 0 && p.nsplit > 0) {
      TileMap map;
      map.per = 0;
      int64_t grid = int64_t(n_int) * p.nsplit;
      const int per = (n_int + 7) / 8;
      if (8 * per <= S_MAXMAP) {
        // interior tiles in 4x4 super-block order, then 8 contiguous chunks
        int order[S_MAXMAP];
        int n = 0;
        const int nsb = (nbf + 3) / 4;
        for (int P = 0; P < nsb; ++P)
          for (int Q = P; Q < nsb; ++Q)
            for (int bi = 4 * P; bi < 4 * P + 4 && bi < nbf; ++bi)
              for (int bj = 4 * Q; bj < 4 * Q + 4 && bj < nbf; ++bj)
                if (bi <= bj) order[n++] = tile_index(bi, bj, p.nb);
        map.per = per;
        for (int i = 0; i < 8 * per; ++i) map.t[i] = 0xffff;
        for (int i = 0; i < n; ++i) map.t[(i / per) * per + i % per] = (unsigned short)order[i];
        grid = int64_t(8) * per * p.nsplit;
      }
      hipLaunchKernelGGL(syrk_f16_lds, dim3(unsigned(grid)), dim3(SY_THREADS), 0, s, Xh, p.n_full, ldx, p.nb, nbf,
                         n_int, p.tokens_per_split, p.nsplit, partial, map);
      if (launch_status() != GPTQ_OK) return GPTQ_E_HIP;
    }
    // Checked path: edge tiles of every split (all tiles when the direct
    // path is unusable), plus the token tail of every tile.
    const int gen_tiles_main = direct ? n_edge : p.ntiles;
    const int64_t n_gen = int64_t(gen_tiles_main) * p.nsplit + (p.nslot > p.nsplit ? p.ntiles : 0);
    if (n_gen > 0) {
      hipLaunchKernelGGL(syrk_f16_generic, dim3(unsigned(n_gen)), dim3(SY_THREADS), 0, s, Xh, n_tokens, p.n_full,
                         int(d), ldx, p.nb, p.ntiles, p.tokens_per_split, p.nsplit, gen_tiles_main,
                         direct ? 0 : 1, partial);
      if (launch_status() != GPTQ_OK) return GPTQ_E_HIP;
    }
  } else {
    hipLaunchKernelGGL(syrk_f32_mfma, dim3(unsigned(int64_t(p.ntiles) * p.nsplit)), dim3(256), 0, s,
                       static_cast<const float*>(X), n_tokens, int(d), ldx, p.nb, p.ntiles, p.tokens_per_split,
                       partial);
    if (launch_status() != GPTQ_OK) return GPTQ_E_HIP;
  }
  const int nob = int((d + 31) / 32);
  hipLaunchKernelGGL(syrk_reduce, dim3(unsigned(nob * (nob + 1) / 2)), dim3(256), 0, s, partial, p.T, p.nb,
                     p.ntiles, p.nslot, int(d), H, accumulate);
  return launch_status();
}
