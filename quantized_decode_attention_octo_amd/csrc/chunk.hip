// octo_attend_chunk: chunk-wise attention over a packed cached window plus a
// full-precision current chunk, on MFMA.
//
// The structure is the cached / current decomposition of chunk-wise video
// diffusion ("Quantized Keys Steal Attention", Sec. 3, Token Structure and
// Attention Decomposition; OCTOPUS paper, Sec. 4.3): every query of the
// current chunk attends, in one softmax and unmasked, to the cached tokens
// (stored with the OCTOPUS codec) and to the current chunk's own keys and
// values.  Everything runs in the rotated frames: q and the current keys are
// rotated by R_k, the current values by R_v; the cached keys and values are
// gamma * u^ straight from the codec (Sec. 3.6, Eq. 13), so that
// (R_k q) . (gamma u^) is the score of the factorized form.  The output is
// R_v^T applied to the softmax-weighted rotated values.
//
// Launches on one stream:
//   1. rotate_rows (x3): q, k_cur -> fp16 rotated rows; v_cur -> fp16 rotated
//      columns of the transposed value matrix
//   2. decode_rows (x2): cached keys -> fp16 gamma u^ rows; cached values ->
//      columns of the transposed value matrix (with the group-wise value
//      codec, Delta code + z, already the rotated value)
//   3. chunk_attn: fp16 MFMA flash attention (fp32 accumulation, online
//      softmax), epilogue 1/l and R_v^T; XCD-aware workgroup order.
// The window is decoded once per call and shared by every query tile.
#include <math.h>

#include <type_traits>

#include "octo_internal.h"

namespace octo {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr float kInvSqrtD = 0.08838834764831845f;
constexpr float kLog2e = 1.4426950408889634f;

// Column of key k in the transposed value matrix.  Within each 32-key block
// the keys are stored in the order in which the score MFMA leaves them in a
// lane's P slots (slot e of lane group g is key 16 (e / 4) + 4 g + e % 4), so
// that a lane's eight value slots are eight consecutive halves: one 16-byte
// LDS read.
__device__ inline int key_column(int k) {
  return (k & ~31) | (((k >> 2) & 3) << 3) | (((k >> 4) & 1) << 2) | (k & 3);
}

// ---------------------------------------------------------------- pre-passes
// Rows t < T_out of a plane: fp16(post H diag(s) x_t), zero for t >= T (tile
// padding); post = 1 / sqrt(d), times the softmax scale and log2(e) for the
// queries, so that scores come out of the MFMA in log2 units.  Row-major
// output: row out_off + t of a [out_rows][128] plane.  Transposed output:
// column key_column(out_off + t) of a [128][out_rows] plane.
// One workgroup takes 64 rows, sixteen lanes a row for the transform; the
// transposed store goes through LDS so that 64 consecutive columns are
// written together.
//
// With `feat` set (queries of the Jensen-bias correction), row t also gets
// kFeat fp16 features: slot j < 128 / feat_gs holds feat_c ||(R x_t)_j||^2
// over group j of the rotated coordinates, the other slots 0.
constexpr int kFeat = 8;           // feature slots per row: groups of g >= 16
struct RotJob {
  const uint16_t* in;            // [planes][T][128] bf16
  int T, T_out;
  uint64_t seed;
  float post;
  _Float16* out;
  int out_rows, out_off;
  _Float16* feat;                // query features, or null
  int feat_gs;
  float feat_c;
  int tiles, planes;             // 64-row tiles per plane; planes (0: no job)
};

template <bool TRANSPOSED>
__device__ inline void rotate_rows(const RotJob& jb, int tile_x, int plane, _Float16* tile) {
  typedef _Float16 half8v __attribute__((ext_vector_type(8)));
  const uint16_t* __restrict__ in = jb.in;
  _Float16* __restrict__ out = jb.out;
  const int T = jb.T, T_out = jb.T_out, out_rows = jb.out_rows, out_off = jb.out_off;
  const uint64_t seed = jb.seed;
  const float post = jb.post;
  _Float16* __restrict__ feat = jb.feat;
  const int feat_gs = jb.feat_gs;
  const float feat_c = jb.feat_c;
  // Sixteen lanes take a row, lane cl holding coordinates 8 cl .. 8 cl + 7
  // (one 16-byte load and store); a wavefront instruction covers 4 rows.
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = lane >> 4, cl = lane & 15;
  const int t0 = tile_x * 64;
  float sg[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) sg[e] = splitmix_sign(seed, 8 * cl + e);
  // the wavefront's 16 rows: every load in flight at once (rows past T read
  // row T - 1 and are zeroed; with T = 0 there is nothing to read)
  uint4 raw[4] = {};
  if (T > 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = min(t0 + 16 * wave + 4 * j + sub, T - 1);
      raw[j] = *reinterpret_cast<const uint4*>(in + ((size_t)plane * T + t) * kHeadDim + 8 * cl);
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int k = 16 * wave + 4 * j + sub, t = t0 + k;
    const uint32_t w[4] = {raw[j].x, raw[j].y, raw[j].z, raw[j].w};
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t h = (e & 1) ? (w[e >> 1] & 0xffff0000u) : (w[e >> 1] << 16);   // bf16 -> fp32
      v[e] = t < T ? __uint_as_float(h) * sg[e] : 0.0f;
    }
    // H (Sylvester order, unnormalized) on the row: coordinate bits 0..2
    // within the lane, bits 3..6 across the row's 16 lanes
#pragma unroll
    for (int m = 1; m < 8; m <<= 1)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (!(e & m)) {
          const float x = v[e], y = v[e | m];
          v[e] = x + y;
          v[e | m] = x - y;
        }
#pragma unroll
    for (int m = 1; m < 16; m <<= 1)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = __shfl_xor(v[e], m, 64);
        v[e] = (cl & m) ? (p - v[e]) : (v[e] + p);
      }
    half8v o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (_Float16)(v[e] * post);
    if (TRANSPOSED) {
      typedef _Float16 half2v __attribute__((ext_vector_type(2)));
#pragma unroll
      for (int e = 0; e < 8; e += 2)
        *reinterpret_cast<half2v*>(&tile[k * 130 + 8 * cl + e]) = half2v{o[e], o[e + 1]};
    } else if (t < T_out) {
      *reinterpret_cast<half8v*>(out + ((size_t)plane * out_rows + out_off + t) * kHeadDim + 8 * cl) = o;
    }
    if (!TRANSPOSED && feat != nullptr) {          // uniform branch
      // group sums of the squared rotated coordinates: a group of feat_gs
      // coordinates is feat_gs / 8 consecutive lanes of the row
      float sq = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) sq = fmaf(v[e] * kInvSqrtD, v[e] * kInvSqrtD, sq);
      const int lpg = feat_gs / 8;
      for (int m = 1; m < lpg; m <<= 1) sq += __shfl_xor(sq, m, 64);
      // slot cl < kFeat of the row's feature vector: group cl, or 0 past the groups
      const int ng = kHeadDim / feat_gs;
      const float f = __shfl(sq, 16 * sub + min(cl, ng - 1) * lpg, 64);
      if (t < T && cl < kFeat) feat[((size_t)plane * T + t) * kFeat + cl] = (_Float16)(cl < ng ? feat_c * f : 0.0f);
    }
  }
  if (TRANSPOSED) {
    __syncthreads();
    for (int e = threadIdx.x; e < 64 * kHeadDim; e += 256) {
      const int c = e >> 6, k = e & 63, t = t0 + k;
      if (t < T_out)
        out[((size_t)plane * kHeadDim + c) * out_rows + key_column(out_off + t)] = tile[k * 130 + c];
    }
  }
}

// The three row transforms of a chunk call (queries; current keys; current
// values, transposed) in one launch, so that the loads of one overlap the
// stores of another: workgroups [0, n0) take job 0, the next n1 job 1, the
// rest job 2, where n_i = tiles_i planes_i.
__global__ __launch_bounds__(256) void rotate_rows_kernel(RotJob q, RotJob k, RotJob v) {
  __shared__ _Float16 tile[64 * 130];
  const int n0 = q.tiles * q.planes, n1 = k.tiles * k.planes;
  int id = blockIdx.x;
  if (id < n0) {
    rotate_rows<false>(q, id % q.tiles, id / q.tiles, tile);
  } else if ((id -= n0) < n1) {
    rotate_rows<false>(k, id % k.tiles, id / k.tiles, tile);
  } else {
    id -= n1;
    rotate_rows<true>(v, id % v.tiles, id / v.tiles, tile);
  }
}

__device__ inline float4 oct_dir(float xi, float eta) {
  const float z = 1.0f - fabsf(xi) - fabsf(eta);
  float x = xi, y = eta;
  if (z < 0.0f) {
    x = (xi >= 0.0f ? 1.0f : -1.0f) * (1.0f - fabsf(eta));
    y = (eta >= 0.0f ? 1.0f : -1.0f) * (1.0f - fabsf(xi));
  }
  const float n = fmaxf(sqrtf(x * x + y * y + z * z), kEps);
  return make_float4(x / n, y / n, z / n, 0.0f);
}

// LDS staging tile of 64 tokens x 128 coordinates, laid out for its store.
// Row-major output: token rows of 130 halves (65 words), so that the 64
// lanes of a wavefront writing one coordinate of 64 tokens meet 64 different
// banks.  Transposed output: coordinate rows of 72 halves holding the tokens
// at key_column order, so that a coordinate's 64 keys leave in 16-byte
// chunks exactly as they lie in the output, and the writes of one coordinate
// fill 32 consecutive words.
template <bool TRANSPOSED>
struct StageTile {
  static constexpr int kRowHalves = TRANSPOSED ? 72 : 130;
  static constexpr int kElems = TRANSPOSED ? kHeadDim * 72 : 64 * 130;
  __device__ static int at(int k, int c) {
    return TRANSPOSED ? c * 72 + key_column(k) : k * 130 + c;
  }
};

// Stores the staging tile of tokens t0 .. t0 + nt - 1 (t0 a multiple of 64)
// as rows of a [out_rows][128] plane (16-byte chunks) or as columns of a
// [128][out_rows] plane at key_column.
template <bool TRANSPOSED>
__device__ inline void store_rows(const _Float16* tile, _Float16* __restrict__ out,
                                  int out_rows, size_t plane, int t0, int nt) {
  const int tid = threadIdx.x;
  if (TRANSPOSED) {
    if (nt == 64) {
      for (int e = tid; e < kHeadDim * 8; e += 256) {
        const int c = e >> 3, q = e & 7;
        *reinterpret_cast<uint4*>(out + (plane * kHeadDim + c) * out_rows + t0 + 8 * q) =
            *reinterpret_cast<const uint4*>(&tile[c * 72 + 8 * q]);
      }
    } else {
      for (int e = tid; e < 64 * kHeadDim; e += 256) {
        const int c = e >> 6, kk = e & 63;
        if (kk < nt)
          out[(plane * kHeadDim + c) * out_rows + key_column(t0 + kk)] =
              tile[StageTile<true>::at(kk, c)];
      }
    }
  } else {
    // four word reads a chunk: token rows are 4-byte but not 16-byte aligned
    const uint32_t* tw = reinterpret_cast<const uint32_t*>(tile);
    for (int e = tid; e < 64 * 16; e += 256) {
      const int kk = e >> 4, c8 = (e & 15) * 8;
      if (kk < nt) {
        const int w0 = kk * 65 + c8 / 2;
        *reinterpret_cast<uint4*>(out + (plane * out_rows + t0 + kk) * kHeadDim + c8) =
            make_uint4(tw[w0], tw[w0 + 1], tw[w0 + 2], tw[w0 + 3]);
      }
    }
  }
}

// One workgroup per 64 cached tokens of a plane: lanes take (token, triplet)
// items token-fastest (coalesced reads of the tile-64 words) and write
// fp16(gamma_t u^_t[0:128]) into an LDS tile, which is then stored as rows t
// of a [out_rows][128] plane (16-byte chunks) or as columns t of a
// [128][out_rows] plane (64 consecutive keys per row, at key_column).
template <int BD, int BN, bool TRANSPOSED>
__global__ __launch_bounds__(256) void decode_rows_kernel(const uint32_t* __restrict__ idx,
                                                          const float* __restrict__ gamma,
                                                          const Codebook cb,
                                                          int capacity, int cached,
                                                          _Float16* __restrict__ out,
                                                          int out_rows) {
  constexpr int K = 1 << BD, R = 1 << BN, FWD = 2 * BD, BT = FWD + BN;
  constexpr int WI = (kNTri * BT + 31) / 32;
  using ST = StageTile<TRANSPOSED>;
  constexpr int kTriG = 11;                        // triplets per thread: 4 x 11 >= 43
  constexpr int GW = (31 + kTriG * BT + 31) / 32;  // record words covering them from any shift
  __shared__ float4 lut[K * K];
  __shared__ float crho[R], cxi[K];
  __shared__ __attribute__((aligned(16))) _Float16 tile[ST::kElems];
  const int tid = threadIdx.x;
  const size_t plane = blockIdx.y;
  const int t0 = blockIdx.x * 64;
  const int nt = min(64, cached - t0);
  // Thread (k, w): token t0 + k, triplets 11 w .. 11 w + 10.  Its record
  // words and gamma are all requested first (a token past the cached ones
  // reads token t0, whose values are not stored).
  const int k = tid & 63, w = tid >> 6;
  const int t = t0 + (k < nt ? k : 0);
  const int iwo = (kTriG * BT * w) >> 5, ish = (kTriG * BT * w) & 31;
  uint32_t wd[GW];
#pragma unroll
  for (int j = 0; j < GW; ++j) wd[j] = idx[tile_word(plane, capacity, t, min(iwo + j, WI - 1), WI)];
  const float gam = gamma[plane * capacity + t];
  if (tid < K) cxi[tid] = cb.xi[tid];
  if (tid < R) crho[tid] = cb.rho[tid];
  __syncthreads();
  for (int e = tid; e < K * K; e += 256) lut[e] = oct_dir(cxi[e % K], cxi[e / K]);
  __syncthreads();
  // shift the words so that triplet 11 w + m starts at bit m B_tri
  uint32_t sw[GW];
#pragma unroll
  for (int j = 0; j < GW; ++j) sw[j] = __builtin_amdgcn_alignbit(j + 1 < GW ? wd[j + 1] : 0u, wd[j], ish);
#pragma unroll
  for (int m = 0; m < kTriG; ++m) {
    const int i = kTriG * w + m;
    if (i >= kNTri) break;
    // triplet field i: code pair | rho index << 2 b_dir
    const uint32_t f = field<BT>(sw, m * BT);
    const uint32_t code = f & ((1u << FWD) - 1u), ir = f >> FWD;
    const float s = crho[ir] * gam;
    const float4 n = lut[code];
    tile[ST::at(k, 3 * i)] = (_Float16)(s * n.x);
    tile[ST::at(k, 3 * i + 1)] = (_Float16)(s * n.y);
    if (i < kNTri - 1) tile[ST::at(k, 3 * i + 2)] = (_Float16)(s * n.z);   // coordinate 128 is the pad
  }
  __syncthreads();
  store_rows<TRANSPOSED>(tile, out, out_rows, plane, t0, nt);
}

// ---------------------------------------------------------------- attention
constexpr int kRG = 2;          // 16-query row groups per wavefront
constexpr int kCWaves = 2;
constexpr int kCThreads = 64 * kCWaves;
constexpr int kBM = 16 * kRG * kCWaves;   // 64 queries per workgroup
constexpr int kXcds = 8;        // workgroups are dealt round-robin to the XCDs
constexpr int kPadKeys = 64;    // the staged key rows are padded to a multiple of this
constexpr float kLazyLog2 = 8.0f;   // slack of the lazy running maximum (log2 units)
// Key tiles: 32 keys per LDS tile, in two buffers: the next tile streams in
// while the current one is used, in 32 KB of LDS (four workgroups per CU).
constexpr int kBN = 32;
constexpr int kVChunks = kBN / 8;                                 // 16-byte chunks per V^T row
constexpr int kTileInsts = kBN * (kHeadDim / 8) / 64 / kCWaves;   // per wavefront, K and V^T each
static_assert(kPadKeys % kBN == 0, "tiles never straddle the padded end");
// LDS tiles are unpadded, written by direct buffer-to-LDS loads (16 bytes a
// lane, 1 KB contiguous per wavefront instruction).  16-byte chunk c of a row
// is stored at chunk c ^ swizzle(row): for key rows (256 B, 16 chunks)
// swizzle = row mod 16, for transposed value rows (64 B, 4 chunks)
// swizzle = (row / 4) mod 4, so that the 16 rows one fragment read touches
// fall in 16 different bank quads.
constexpr int kKChunks = kHeadDim / 8;   // 16-byte chunks per key row
// Fourth word of a raw buffer descriptor: 32-bit data format, no swizzle.
constexpr int kBufferWord3 = 0x00020000;
// s_waitcnt immediate waiting until no vector-memory operation of the
// wavefront is outstanding (vmcnt 0; expcnt and lgkmcnt not waited for).
constexpr int kWaitVm0 = (0x7 << 4) | (0xF << 8);

struct ChunkArgs {
  const _Float16* q;   // [B][Hq][Tq][128] rotated, times scale log2(e)
  const _Float16* k;   // [B][Hkv][Tk_pad][128] rotated
  const _Float16* vt;  // [B][Hkv][128][Tk_pad] rotated, transposed
  float* out;          // [B][Hq][Tq][128]
  int Hq, Hkv, Tq, Tk, Tk_pad;
  int q_tiles;         // query tiles per (batch, head)
  uint64_t vseed;
  // Jensen-bias correction: fp16 feature rows whose product is minus the
  // bias in log2 units ([B][Hq][Tq][kFeat] queries, [B][Hkv][Tk_pad][kFeat] keys)
  const _Float16* qfeat;
  const _Float16* kfeat;
};

// Lane layout of v_mfma_f32_16x16x32_f16 (wave of 64, L = lane):
//   A[i][k]: i = L % 16, k = 8 (L / 16) + e  (e = element 0..7)
//   B[k][j]: j = L % 16, k = 8 (L / 16) + e
//   D[i][j]: i = 4 (L / 16) + r, j = L % 16  (r = register 0..3)
// Scores are computed transposed, S^T = K Q^T (keys are rows), so that each
// lane ends up with 4 keys of one query, which is exactly the A operand
// layout P needs for O = P V with keys as the contraction index.  Each
// wavefront owns two 16-query row groups, so every key / value fragment read
// from LDS feeds two MFMAs.  The softmax state is updated once per 64-key
// tile.  Small workgroups (64 queries) keep four resident per CU, which
// hides the tile loads and leaves no lone final round of workgroups.
//
// XCD-aware order: the hardware deals consecutive workgroup ids to the 8
// XCDs in turn, so the linear id is mapped such that all query tiles of one
// (batch, head) run on the same XCD and stream its keys and values through
// that XCD's L2 together.
//
// CORR: the Jensen-bias correction ("Quantized Keys Steal Attention",
// Eq. 15).  Its bias is a rank-(128 / g) product of query and key features,
// so it is one more k-slice of the score MFMA per 16 keys, whose slots 0..7
// (lane group 0) hold the features and the rest zeros: lane group 0 reads
// the tile's key features (beside the tile, 512 B a buffer) and the
// workgroup's query features (1 KB of LDS) where they are used, the other
// lanes hold zeros, so four workgroups still share a CU.
template <bool CORR>
__global__ __launch_bounds__(kCThreads, 2) void chunk_attn_kernel(ChunkArgs a) {
  __shared__ __attribute__((aligned(1024))) _Float16 ks0[kBN * kHeadDim], ks1[kBN * kHeadDim];
  __shared__ __attribute__((aligned(1024))) _Float16 vs0[kHeadDim * kBN], vs1[kHeadDim * kBN];
  __shared__ __attribute__((aligned(1024))) _Float16 kfs0[CORR ? kBN * kFeat : 8],
      kfs1[CORR ? kBN * kFeat : 8];
  __shared__ _Float16 qfs[CORR ? kBM * kFeat : 1];
  const int tid = threadIdx.x, L = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = L & 15, grp = L >> 4;
  const int n_units = gridDim.x;
  const int id = blockIdx.x;
  // id -> (xcd, local); units (head-major, tile-minor) are split into 8
  // contiguous ranges, range x running on XCD x.
  const int per_xcd = (n_units + kXcds - 1) / kXcds;
  const int xcd = id % kXcds, local = id / kXcds;
  const int full_xcds = n_units - (per_xcd - 1) * kXcds;   // XCDs with per_xcd units
  const int unit = xcd < full_xcds ? xcd * per_xcd + local
                                   : full_xcds * per_xcd + (xcd - full_xcds) * (per_xcd - 1) + local;
  const int tile = unit % a.q_tiles, bh = unit / a.q_tiles;
  const int hq = bh % a.Hq, b = bh / a.Hq;
  const int hk = hq / (a.Hq / a.Hkv);
  const int q0 = tile * kBM + wave * 16 * kRG;
  if constexpr (CORR) {
    // the workgroup's 64 query feature rows (rows past Tq repeat the last)
    for (int r = tid; r < kBM; r += kCThreads) {
      const int qrow = min(tile * kBM + r, a.Tq - 1);
      *reinterpret_cast<half8*>(&qfs[r * kFeat]) = *reinterpret_cast<const half8*>(
          a.qfeat + (((size_t)b * a.Hq + hq) * a.Tq + qrow) * kFeat);
    }
  }

  // Q^T fragments (B operand): query q0 + 16 rg + col, dims 32 s + 8 grp + e.
  half8 qf[kRG][4];
#pragma unroll
  for (int rg = 0; rg < kRG; ++rg) {
    const int qrow = min(q0 + 16 * rg + col, a.Tq - 1);
    const _Float16* src = a.q + (((size_t)b * a.Hq + hq) * a.Tq + qrow) * kHeadDim;
#pragma unroll
    for (int s = 0; s < 4; ++s) qf[rg][s] = *reinterpret_cast<const half8*>(src + 32 * s + 8 * grp);
  }
  floatx4 o[kRG][8];
#pragma unroll
  for (int rg = 0; rg < kRG; ++rg)
#pragma unroll
    for (int c = 0; c < 8; ++c) o[rg][c] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  // of query q0 + 16 rg + col: running maximum (log2 units), and this
  // lane's part of the normalizer
  float m_run[kRG], l_run[kRG];
#pragma unroll
  for (int rg = 0; rg < kRG; ++rg) {
    m_run[rg] = -INFINITY;
    l_run[rg] = 0.0f;
  }

  const size_t kbase = ((size_t)b * a.Hkv + hk) * a.Tk_pad * kHeadDim;
  const size_t vbase = ((size_t)b * a.Hkv + hk) * kHeadDim * a.Tk_pad;
  // The tiles of K (kBN rows x 128 dims, contiguous) and V^T (128 rows x kBN
  // keys) go straight from global memory to LDS: wavefront w issues
  // instructions j < kTileInsts of each, lane L of instruction j filling
  // stored chunk p = 64 (kTileInsts w + j) + L, i.e. row p / 16 (K) or
  // p / kVChunks (V^T), whose logical chunk is the stored one xor the row's
  // swizzle.  Every load of a tile is in flight at once and holds no registers.
  static_assert(kCWaves * kTileInsts * 64 == kBN * kKChunks &&
                    kCWaves * kTileInsts * 64 == kHeadDim * kVChunks,
                "the wavefronts' instructions fill each tile");
  // The swizzle of instruction j depends on j mod 4 (K) and j mod 2 (V^T):
  // a lane keeps four and two source offsets, the rest are uniform steps.
  uint32_t ksrc[4], vsrc[2];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int p = 64 * (kTileInsts * wave + j) + L;
    const int kr = p / kKChunks, kc = (p % kKChunks) ^ (kr % kKChunks);
    ksrc[j] = (uint32_t)((kr * kHeadDim + kc * 8) * 2);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int p = 64 * (kTileInsts * wave + j) + L;
    const int vr = p / kVChunks, vc = (p % kVChunks) ^ ((vr / (16 / kVChunks)) % kVChunks);
    vsrc[j] = (uint32_t)(vr * a.Tk_pad * 2 + vc * 16);
  }
  const int vstep = (128 / kVChunks) * a.Tk_pad * 2;   // two instructions' rows, in bytes
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<_Float16*>(a.k + kbase), (short)0, a.Tk_pad * kHeadDim * 2, kBufferWord3);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<_Float16*>(a.vt + vbase), (short)0, a.Tk_pad * kHeadDim * 2, kBufferWord3);
  const __amdgpu_buffer_rsrc_t frs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<_Float16*>(CORR ? a.kfeat + ((size_t)b * a.Hkv + hk) * a.Tk_pad * kFeat : a.k),
      (short)0, a.Tk_pad * kFeat * 2, kBufferWord3);
  // Issues the loads of the tile at kt0 into (ks, vs, kfs); none is waited for here.
  auto copy_tile = [&](int kt0, _Float16* ks, _Float16* vs, _Float16* kfs) {
#pragma unroll
    for (int j = 0; j < kTileInsts; ++j) {
      const int inst = kTileInsts * wave + j;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, ks + 512 * inst, 16, ksrc[j & 3],
                                               kt0 * kHeadDim * 2 + (j >> 2) * 4096, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, vs + 512 * inst, 16, vsrc[j & 1],
                                               kt0 * 2 + (j >> 1) * vstep, 0, 0);
    }
    if constexpr (CORR) {
      // the tile's key feature rows, a 16-byte row a lane of wavefront 0
      if (wave == 0 && L < kBN)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(frs, kfs, 16, L * kFeat * 2, kt0 * kFeat * 2, 0, 0);
    }
  };

  // One tile from LDS; only the last, ragged tile masks keys past Tk.
  auto tile_step = [&](int kt0, auto masked_c, const _Float16* ks, const _Float16* vs,
                       const _Float16* kfs) {
    constexpr bool MASKED = decltype(masked_c)::value;
    // scores of the tile's keys (log2 units): st[kt][rg][r] = key kt0 + 16 kt + 4 grp + r
    floatx4 st[kBN / 16][kRG];
    const half8 zero8 = {};
#pragma unroll
    for (int kt = 0; kt < kBN / 16; ++kt) {
#pragma unroll
      for (int rg = 0; rg < kRG; ++rg) st[kt][rg] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
      // key 16 kt + col (row swizzle col), logical chunk 4 s + grp
      const _Float16* kr = &ks[(16 * kt + col) * kHeadDim];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const half8 kf = *reinterpret_cast<const half8*>(kr + 8 * ((4 * s + grp) ^ col));
#pragma unroll
        for (int rg = 0; rg < kRG; ++rg)
          st[kt][rg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, qf[rg][s], st[kt][rg], 0, 0, 0);
      }
      if constexpr (CORR) {
        // minus the Jensen bias of keys 16 kt + (0..15), in log2 units
        // (slots 8..31 of both operands are zero: lane groups 1..3 read nothing)
        half8 kf5 = zero8;
        if (grp == 0) kf5 = *reinterpret_cast<const half8*>(&kfs[(16 * kt + col) * kFeat]);
#pragma unroll
        for (int rg = 0; rg < kRG; ++rg) {
          half8 qf5 = zero8;
          if (grp == 0)
            qf5 = *reinterpret_cast<const half8*>(&qfs[(wave * 16 * kRG + 16 * rg + col) * kFeat]);
          st[kt][rg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf5, qf5, st[kt][rg], 0, 0, 0);
        }
      }
    }
    half8 pf[kRG][kBN / 32];
#pragma unroll
    for (int rg = 0; rg < kRG; ++rg) {
      float x[kBN / 4];
      float mx = -INFINITY;
#pragma unroll
      for (int e = 0; e < kBN / 4; ++e) {
        const int kt = e >> 2, r = e & 3;
        x[e] = st[kt][rg][r];
        if (MASKED && kt0 + 16 * kt + 4 * grp + r >= a.Tk) x[e] = -INFINITY;
        mx = fmaxf(mx, x[e]);
      }
      mx = rows_max(mx);
      // Lazy running maximum: a row moves its maximum (and rescales its sums)
      // only when a score exceeds it by more than kLazyLog2, so that nearly
      // every tile skips the rescale; probabilities then stay below
      // 2^kLazyLog2, well inside fp16, and the final 1/l cancels the shift.
      const bool up = mx > m_run[rg] + kLazyLog2;
      if (__ballot(up)) {
        const float m_new = up ? mx : m_run[rg];
        const float alpha = up ? __builtin_amdgcn_exp2f(m_run[rg] - m_new) : 1.0f;
        l_run[rg] *= alpha;
        m_run[rg] = m_new;
        // rescale O rows (queries q0 + 16 rg + 4 grp + r)
        float al[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) al[r] = __shfl(alpha, 4 * grp + r, 64);
#pragma unroll
        for (int c = 0; c < 8; ++c)
#pragma unroll
          for (int r = 0; r < 4; ++r) o[rg][c][r] *= al[r];
      }
      float ps = 0.0f;
#pragma unroll
      for (int e = 0; e < kBN / 4; ++e) {
        // the raw exp2 (flushing results below the normal range to zero) is
        // exact enough next to the row's largest terms (at least 1)
        const float p = __builtin_amdgcn_exp2f(x[e] - m_run[rg]);
        ps += p;
        pf[rg][e >> 3][e & 7] = (_Float16)p;
      }
      l_run[rg] += ps;                 // this lane's keys; rows are summed at the end
    }
    // O += P V: slot e of sub-block sb is key kt0 + 32 sb + 16 (e / 4) + 4 grp + e % 4
#pragma unroll
    for (int sb = 0; sb < kBN / 32; ++sb)
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        // value row 16 c + col, logical chunk 4 sb + grp
        const int sw = (col / (16 / kVChunks)) % kVChunks;
        const half8 vf = *reinterpret_cast<const half8*>(
            &vs[(16 * c + col) * kBN + 8 * ((4 * sb + grp) ^ sw)]);
#pragma unroll
        for (int rg = 0; rg < kRG; ++rg)
          o[rg][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pf[rg][sb], vf, o[rg][c], 0, 0, 0);
      }
  };
  const int tk_full = a.Tk / kBN * kBN;
  const int n_tiles = (a.Tk + kBN - 1) / kBN;
  auto compute = [&](int t, const _Float16* ks, const _Float16* vs, const _Float16* kfs) {
    if (t * kBN < tk_full)
      tile_step(t * kBN, std::false_type{}, ks, vs, kfs);
    else
      tile_step(t * kBN, std::true_type{}, ks, vs, kfs);
  };
  // Tile t sits in buffer t % 2.  Tile t + 1 is requested before tile t's
  // arithmetic and waited for after it, at the barrier (whose fence also
  // waits for this wave's loads into LDS), which also frees buffer t % 2.
  auto step = [&](int t, const _Float16* ks, const _Float16* vs, const _Float16* kfs,
                  _Float16* nks, _Float16* nvs, _Float16* nkfs) {
    if (t + 1 < n_tiles) copy_tile((t + 1) * kBN, nks, nvs, nkfs);
    compute(t, ks, vs, kfs);
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    lds_barrier();
  };
  if (n_tiles > 0) copy_tile(0, ks0, vs0, kfs0);
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  lds_barrier();
  for (int t = 0; t < n_tiles; t += 2) {
    step(t, ks0, vs0, kfs0, ks1, vs1, kfs1);
    if (t + 1 < n_tiles) step(t + 1, ks1, vs1, kfs1, ks0, vs0, kfs0);
  }

  // ---- epilogue: 1/l, then R_v^T = diag(s_v) H / sqrt(d) on every query row.
  // Lane holds coordinate 16 c + col of queries q0 + 16 rg + 4 grp + r: the
  // Hadamard butterflies on coordinate bits 4..6 are register-local, bits
  // 0..3 cross lanes within each 16-lane group.
  float sv[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) sv[c] = kInvSqrtD * splitmix_sign(a.vseed, 16 * c + col);
#pragma unroll
  for (int rg = 0; rg < kRG; ++rg) {
    const float l_tot = rows_sum(l_run[rg]);   // the row's four lane groups
    float li[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float l = __shfl(l_tot, 4 * grp + r, 64);
      li[r] = l > 0.0f ? 1.0f / l : 0.0f;
    }
    float v[8][4];
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r) v[c][r] = o[rg][c][r] * li[r];
#pragma unroll
    for (int m = 4; m >= 1; m >>= 1)
#pragma unroll
      for (int c = 0; c < 8; ++c)
        if (!(c & m)) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float x = v[c][r], y = v[c | m][r];
            v[c][r] = x + y;
            v[c | m][r] = x - y;
          }
        }
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1)
#pragma unroll
      for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = __shfl_xor(v[c][r], m, 64);
          v[c][r] = (col & m) ? (p - v[c][r]) : (v[c][r] + p);
        }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int q = q0 + 16 * rg + 4 * grp + r;
      if (q >= a.Tq) continue;
      float* dst = a.out + (((size_t)b * a.Hq + hq) * a.Tq + q) * kHeadDim;
#pragma unroll
      for (int c = 0; c < 8; ++c) dst[16 * c + col] = v[c][r] * sv[c];
    }
  }
}

// The group-wise value codec: one workgroup per 64 cached tokens of a plane
// stages their records (word w of the 64 tokens is 256 contiguous bytes) in
// LDS, then thread (token, quarter) writes fp16(Delta code + z), the rotated
// value, of its 32 coordinates into the tile stored as above.
template <int VB, int GS, bool TRANSPOSED>
__global__ __launch_bounds__(256) void group_decode_rows_kernel(const uint32_t* __restrict__ idx,
                                                                int capacity, int cached,
                                                                _Float16* __restrict__ out,
                                                                int out_rows) {
  constexpr int G = kHeadDim / GS, WC = VB * kHeadDim / 32, W = group_record_words(VB, GS);
  using ST = StageTile<TRANSPOSED>;
  __shared__ uint32_t rec[W * 64];
  __shared__ __attribute__((aligned(16))) _Float16 tile[ST::kElems];
  const int tid = threadIdx.x;
  const size_t plane = blockIdx.y;
  const int t0 = blockIdx.x * 64;
  const int nt = min(64, cached - t0);
  // every load of the staging goes out before the first LDS store
  constexpr int kLoads = (W * 64 + 255) / 256;
  uint32_t rv[kLoads];
#pragma unroll
  for (int j = 0; j < kLoads; ++j) {
    const int e = tid + 256 * j, w = e >> 6, k = e & 63;
    rv[j] = e < W * 64 && k < nt ? idx[tile_word(plane, capacity, t0 + k, w, W)] : 0u;
  }
#pragma unroll
  for (int j = 0; j < kLoads; ++j) {
    const int e = tid + 256 * j;
    if (e < W * 64) rec[e] = rv[j];
  }
  __syncthreads();
  // Thread (k, w): token k, coordinates 32 w .. 32 w + 31, whose codes fill
  // words VB w .. VB w + VB - 1 of the record and whose groups' steps and
  // zero points are decoded once.
  static_assert(GS == 16 || GS == 32, "a thread's 32 coordinates span whole groups");
  const int k = tid & 63, w = tid >> 6;
  uint32_t cw[VB];
#pragma unroll
  for (int i = 0; i < VB; ++i) cw[i] = rec[(VB * w + i) * 64 + k];
#pragma unroll
  for (int gi = 0; gi < 32 / GS; ++gi) {
    const int j = (32 / GS) * w + gi;
    const uint32_t sw = rec[(WC + j / 4) * 64 + k], zw = rec[(WC + G / 4 + j / 2) * 64 + k];
    const float dh = e4m3_value((sw >> (8 * (j % 4))) & 0xffu);
    const float zh = __uint_as_float(((zw >> (16 * (j % 2))) & 0xffffu) << 16);
#pragma unroll
    for (int m = 0; m < GS; ++m) {
      const int cl = GS * gi + m;
      const uint32_t q = field<VB>(cw, cl * VB);
      tile[ST::at(k, 32 * w + cl)] = (_Float16)fmaf(dh, (float)q, zh);
    }
  }
  __syncthreads();
  store_rows<TRANSPOSED>(tile, out, out_rows, plane, t0, nt);
}

// Key features of the Jensen-bias correction: row t < Tk_pad of a plane gets
// Delta^_tj^2 / 16 in slot j < 128 / GS for the cached tokens (t < cached),
// 0 elsewhere (current tokens, tile padding, unused slots).  The factor 1/16
// keeps Delta^2 <= 448^2 in the fp16 range; the query features carry 16.
template <int VB, int GS>
__global__ __launch_bounds__(256) void key_features_kernel(const uint32_t* __restrict__ idx,
                                                           int capacity, int cached, int Tk_pad,
                                                           _Float16* __restrict__ feat) {
  constexpr int G = kHeadDim / GS, WC = VB * kHeadDim / 32, W = group_record_words(VB, GS);
  const size_t plane = blockIdx.y;
  const int t0 = blockIdx.x * 64;
  for (int e = threadIdx.x; e < 64 * kFeat; e += 256) {
    const int t = t0 + e / kFeat, j = e % kFeat;
    float f = 0.0f;
    if (t < cached && j < G) {
      const uint32_t sw = idx[tile_word(plane, capacity, t, WC + j / 4, W)];
      const float dh = e4m3_value((sw >> (8 * (j % 4))) & 0xffu);
      f = dh * dh * 0.0625f;
    }
    feat[(plane * Tk_pad + t) * kFeat + j] = (_Float16)f;
  }
}

struct ChunkPlan {
  int Tk, Tk_pad;
  size_t q_off, k_off, v_off, qf_off, kf_off, total;
};

// corr: room for the correction's query and key feature rows after the rows
ChunkPlan chunk_plan(int B, int Hq, int Hkv, int Tq, int cached, int Tc, bool corr) {
  ChunkPlan p;
  p.Tk = cached + Tc;
  p.Tk_pad = (p.Tk + kPadKeys - 1) / kPadKeys * kPadKeys;
  const size_t row = kHeadDim * sizeof(_Float16);
  auto up = [](size_t n) { return (n + 255) / 256 * 256; };
  p.q_off = 0;
  p.k_off = up((size_t)B * Hq * Tq * row);
  const size_t kv = (size_t)B * Hkv * p.Tk_pad * row;
  p.v_off = p.k_off + up(kv);
  p.total = p.v_off + kv;
  p.qf_off = p.kf_off = 0;
  if (corr) {
    const size_t frow = kFeat * sizeof(_Float16);
    p.qf_off = up(p.total);
    p.kf_off = p.qf_off + up((size_t)B * Hq * Tq * frow);
    p.total = p.kf_off + (size_t)B * Hkv * p.Tk_pad * frow;
  }
  return p;
}

template <int BD, int BN>
void launch_decode_rows(const octo_cache_view* c, const Codec& cd, int cached, _Float16* out,
                        int out_rows, bool transposed, hipStream_t st) {
  dim3 grid((cached + 63) / 64, c->batch * c->kv_heads);
  if (transposed)
    hipLaunchKernelGGL((decode_rows_kernel<BD, BN, true>), grid, dim3(256), 0, st, c->idx,
                       c->gamma, cd.cb, c->capacity, cached, out, out_rows);
  else
    hipLaunchKernelGGL((decode_rows_kernel<BD, BN, false>), grid, dim3(256), 0, st, c->idx,
                       c->gamma, cd.cb, c->capacity, cached, out, out_rows);
}

template <int VB, int GS>
void launch_group_rows(const octo_cache_view* c, int cached, _Float16* out, int out_rows,
                       bool transposed, hipStream_t st) {
  dim3 grid((cached + 63) / 64, c->batch * c->kv_heads);
  if (transposed)
    hipLaunchKernelGGL((group_decode_rows_kernel<VB, GS, true>), grid, dim3(256), 0, st, c->idx,
                       c->capacity, cached, out, out_rows);
  else
    hipLaunchKernelGGL((group_decode_rows_kernel<VB, GS, false>), grid, dim3(256), 0, st, c->idx,
                       c->capacity, cached, out, out_rows);
}

bool decode_rows(const octo_cache_view* c, const Codec& cd, int cached, _Float16* out,
                 int out_rows, bool transposed, hipStream_t st) {
  if (cd.group) {
    switch (cd.bits * 100 + cd.group) {
      case 216: launch_group_rows<2, 16>(c, cached, out, out_rows, transposed, st); return true;
      case 232: launch_group_rows<2, 32>(c, cached, out, out_rows, transposed, st); return true;
      case 316: launch_group_rows<3, 16>(c, cached, out, out_rows, transposed, st); return true;
      case 332: launch_group_rows<3, 32>(c, cached, out, out_rows, transposed, st); return true;
      case 416: launch_group_rows<4, 16>(c, cached, out, out_rows, transposed, st); return true;
      case 432: launch_group_rows<4, 32>(c, cached, out, out_rows, transposed, st); return true;
    }
    return false;
  }
  switch (cd.b_dir * 10 + cd.b_nrm) {
    case 31: launch_decode_rows<3, 1>(c, cd, cached, out, out_rows, transposed, st); return true;
    case 42: launch_decode_rows<4, 2>(c, cd, cached, out, out_rows, transposed, st); return true;
    case 53: launch_decode_rows<5, 3>(c, cd, cached, out, out_rows, transposed, st); return true;
    case 22: launch_decode_rows<2, 2>(c, cd, cached, out, out_rows, transposed, st); return true;
    case 33: launch_decode_rows<3, 3>(c, cd, cached, out, out_rows, transposed, st); return true;
    case 44: launch_decode_rows<4, 4>(c, cd, cached, out, out_rows, transposed, st); return true;
  }
  return false;
}

}  // namespace
}  // namespace octo

using namespace octo;

extern "C" octo_status octo_chunk_workspace_bytes(const octo_codec_desc* k_codec, int32_t B,
                                                  int32_t num_q_heads, int32_t kv_heads,
                                                  int32_t Tq, int32_t cached_tokens, int32_t Tc,
                                                  uint32_t flags, size_t* bytes) {
  clear_error();
  Codec kc;
  octo_status s = resolve_codec(k_codec, "octo_chunk_workspace_bytes", &kc, false);
  if (s != OCTO_OK) return s;
  if (flags & ~OCTO_CHUNK_JENSEN_CORRECTION)
    return fail(OCTO_ERR_INVALID_ARGUMENT, "octo_chunk_workspace_bytes: unknown flags 0x%x", flags);
  if (!bytes) return fail(OCTO_ERR_INVALID_ARGUMENT, "octo_chunk_workspace_bytes: bytes is NULL");
  if (B < 1 || num_q_heads < 1 || kv_heads < 1 || Tq < 0 || cached_tokens < 0 || Tc < 0)
    return fail(OCTO_ERR_INVALID_ARGUMENT, "octo_chunk_workspace_bytes: bad sizes");
  *bytes = chunk_plan(B, num_q_heads, kv_heads, Tq, cached_tokens, Tc,
                      (flags & OCTO_CHUNK_JENSEN_CORRECTION) != 0).total;
  return OCTO_OK;
}

extern "C" octo_status octo_attend_chunk(const octo_codec_desc* k_codec,
                                         const octo_codec_desc* v_codec,
                                         const octo_cache_view* k_cache,
                                         const octo_cache_view* v_cache, int32_t cached_tokens,
                                         const void* q, const void* k_cur, const void* v_cur,
                                         int32_t num_q_heads, int32_t Tq, int32_t Tc,
                                         float softmax_scale, uint32_t flags, float* out,
                                         void* workspace, size_t workspace_bytes,
                                         hipStream_t stream) {
  clear_error();
  const char* what = "octo_attend_chunk";
  Codec kc, vc;
  octo_status s;
  if ((s = resolve_codec(k_codec, what, &kc)) != OCTO_OK) return s;
  if ((s = resolve_codec(v_codec, what, &vc)) != OCTO_OK) return s;
  if ((s = check_cache(k_cache, kc, what)) != OCTO_OK) return s;
  if ((s = check_cache(v_cache, vc, what)) != OCTO_OK) return s;
  if (kc.qjl || vc.qjl) return fail(OCTO_ERR_UNSUPPORTED, "%s: QJL is not supported here", what);
  if (flags & ~OCTO_CHUNK_JENSEN_CORRECTION)
    return fail(OCTO_ERR_INVALID_ARGUMENT, "%s: unknown flags 0x%x", what, flags);
  const bool corr = (flags & OCTO_CHUNK_JENSEN_CORRECTION) != 0;
  if (corr && !kc.group)
    return fail(OCTO_ERR_UNSUPPORTED,
                "%s: the Jensen-bias correction models round-to-nearest keys (group codec)", what);
  if (k_cache->batch != v_cache->batch || k_cache->kv_heads != v_cache->kv_heads ||
      k_cache->capacity != v_cache->capacity)
    return fail(OCTO_ERR_INVALID_ARGUMENT, "%s: K and V caches differ in shape", what);
  const int B = k_cache->batch, Hkv = k_cache->kv_heads;
  if (num_q_heads < 1 || num_q_heads % Hkv)
    return fail(OCTO_ERR_INVALID_ARGUMENT, "%s: %d query heads on %d KV heads", what,
                num_q_heads, Hkv);
  if (Tq < 0 || Tc < 0 || cached_tokens < 0)
    return fail(OCTO_ERR_INVALID_ARGUMENT, "%s: negative size", what);
  if (cached_tokens > k_cache->capacity)
    return fail(OCTO_ERR_CAPACITY, "%s: cached_tokens %d > capacity %d", what, cached_tokens,
                k_cache->capacity);
  if (B > 65535 || num_q_heads > 65535)
    return fail(OCTO_ERR_UNSUPPORTED, "%s: batch and heads must be <= 65535", what);
  if (Tq == 0) return OCTO_OK;
  if (!q || !out || (Tc > 0 && (!k_cur || !v_cur)))
    return fail(OCTO_ERR_INVALID_ARGUMENT, "%s: q, out, k_cur, v_cur must be set", what);
  // the rows are read 16 bytes a lane
  if (((uintptr_t)q | (uintptr_t)k_cur | (uintptr_t)v_cur) & 15 || ((uintptr_t)out & 3))
    return fail(OCTO_ERR_ALIGNMENT, "%s: q, k_cur, v_cur (16 bytes) or out (4) misaligned", what);
  const ChunkPlan p = chunk_plan(B, num_q_heads, Hkv, Tq, cached_tokens, Tc, corr);
  // the attention kernel addresses a plane's staged keys and values through
  // buffer descriptors with 32-bit byte ranges
  if ((int64_t)p.Tk_pad * kHeadDim * 2 > INT32_MAX)
    return fail(OCTO_ERR_UNSUPPORTED, "%s: %d keys a plane exceed 2 GiB of staged rows", what,
                p.Tk_pad);
  if (!workspace || workspace_bytes < p.total)
    return fail(OCTO_ERR_WORKSPACE_TOO_SMALL, "%s: workspace %zu bytes, need %zu", what,
                workspace_bytes, p.total);
  if ((uintptr_t)workspace & 255)
    return fail(OCTO_ERR_ALIGNMENT, "%s: workspace must be 256-byte aligned", what);

  char* ws = static_cast<char*>(workspace);
  _Float16* qr = reinterpret_cast<_Float16*>(ws + p.q_off);
  _Float16* kr = reinterpret_cast<_Float16*>(ws + p.k_off);
  _Float16* vr = reinterpret_cast<_Float16*>(ws + p.v_off);
  const int planes_q = B * num_q_heads, planes_kv = B * Hkv;

  const float tau = softmax_scale > 0.0f ? softmax_scale : kInvSqrtD;
  const float scale2 = tau * kLog2e;
  _Float16* qf = corr ? reinterpret_cast<_Float16*>(ws + p.qf_off) : nullptr;
  _Float16* kf = corr ? reinterpret_cast<_Float16*>(ws + p.kf_off) : nullptr;
  // query features: minus 16 log2(e) tau^2 / 24 ||(R q)_j||^2 (the key
  // features carry Delta^2 / 16), so that their product is -b in log2 units
  const float feat_c = -16.0f * kLog2e * tau * tau / 24.0f;
  RotJob jq{static_cast<const uint16_t*>(q), Tq, Tq, kc.seed, kInvSqrtD * scale2, qr, Tq, 0,
            qf, corr ? kc.group : 32, feat_c, (Tq + 63) / 64, planes_q};
  const int cur_out = p.Tk_pad - cached_tokens;  // current rows plus the zero tile padding
  const int cur_tiles = cur_out > 0 ? (cur_out + 63) / 64 : 0;
  RotJob jk{static_cast<const uint16_t*>(k_cur), Tc, cur_out, kc.seed, kInvSqrtD, kr, p.Tk_pad,
            cached_tokens, nullptr, 32, 0.0f, cur_tiles, planes_kv};
  RotJob jv{static_cast<const uint16_t*>(v_cur), Tc, cur_out, vc.seed, kInvSqrtD, vr, p.Tk_pad,
            cached_tokens, nullptr, 32, 0.0f, cur_tiles, planes_kv};
  const long rot_blocks = (long)jq.tiles * jq.planes + 2L * cur_tiles * planes_kv;
  if (rot_blocks > 0)
    hipLaunchKernelGGL(rotate_rows_kernel, dim3((unsigned)rot_blocks), dim3(256), 0, stream, jq, jk, jv);
  if (cached_tokens > 0) {
    if (!decode_rows(k_cache, kc, cached_tokens, kr, p.Tk_pad, false, stream) ||
        !decode_rows(v_cache, vc, cached_tokens, vr, p.Tk_pad, true, stream))
      return fail(OCTO_ERR_UNSUPPORTED, "%s: split not compiled", what);
  }
  if (corr && p.Tk_pad > 0) {
    const dim3 fgrid(p.Tk_pad / 64, planes_kv);
    switch (kc.bits * 100 + kc.group) {
#define OCTO_KEY_FEATURES(VB, GS)                                                            \
  hipLaunchKernelGGL((key_features_kernel<VB, GS>), fgrid, dim3(256), 0, stream, k_cache->idx, \
                     k_cache->capacity, cached_tokens, p.Tk_pad, kf)
      case 216: OCTO_KEY_FEATURES(2, 16); break;
      case 232: OCTO_KEY_FEATURES(2, 32); break;
      case 316: OCTO_KEY_FEATURES(3, 16); break;
      case 332: OCTO_KEY_FEATURES(3, 32); break;
      case 416: OCTO_KEY_FEATURES(4, 16); break;
      case 432: OCTO_KEY_FEATURES(4, 32); break;
#undef OCTO_KEY_FEATURES
      default: return fail(OCTO_ERR_UNSUPPORTED, "%s: group codec not compiled", what);
    }
  }
  if ((s = check_launch(what)) != OCTO_OK) return s;
  ChunkArgs a;
  a.q = qr;
  a.k = kr;
  a.vt = vr;
  a.out = out;
  a.Hq = num_q_heads;
  a.Hkv = Hkv;
  a.Tq = Tq;
  a.Tk = p.Tk;
  a.Tk_pad = p.Tk_pad;
  a.q_tiles = (Tq + kBM - 1) / kBM;
  a.vseed = vc.seed;
  a.qfeat = qf;
  a.kfeat = kf;
  const long long units = (long long)a.q_tiles * num_q_heads * B;
  if (units > 0x7fffffffLL)
    return fail(OCTO_ERR_UNSUPPORTED, "%s: too many query tiles", what);
  if (corr)
    hipLaunchKernelGGL(chunk_attn_kernel<true>, dim3((unsigned)units), dim3(kCThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(chunk_attn_kernel<false>, dim3((unsigned)units), dim3(kCThreads), 0, stream, a);
  return check_launch(what);
}
