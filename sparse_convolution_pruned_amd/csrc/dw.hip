// Weight and bias gradients as a split-K reduction over tokens.
//   dW[j][i][o] = sum_k X[N[k,j]][i] dY[k][o]      (a GEMM with M = taps C_in,
//   db[o]       = sum_k dY[k][o]                     N = C_out, K = tokens)
// for a K x K neighbourhood with taps = K * K (9 in the page's 3 x 3 case).
// ("SV-TAD: Native Sparse Convolutions for Efficient Temporal Action
// Detection", Key Design 2 names dedicated backward kernels; the formula is
// the adjoint of the forward sum.)
//
// The token range is cut into slices; each slice writes fp32 partial sums to
// the workspace and a final pass adds the slices in ascending order, so the
// result is bitwise reproducible.  With one slice the partial kernel writes
// dW directly.
//
// The MFMA kernel (bf16, C_in and C_out multiples of 128) is described
// below; other shapes and fp32 use the VALU kernel in conv_valu.hip.
#include <type_traits>

#include "internal.h"
#include "mfma.h"

namespace svc {

hipError_t launch_dw_valu(bool bf16, const void* X, const int32_t* N, const void* dY, float* out,
                          int64_t n, int Ci, int Co, int taps, int slices, int64_t slice_tokens,
                          int direct, int accumulate, hipStream_t stream);

// MFMA kernel.  A unit is one (tap, 128-input-channel tile) pair; units are
// numbered tap-fastest (u = tile * taps + tap) and cut into groups of three,
// the last group padded with empty units.  At 3 x 3 a group is one kernel
// row (taps 3r, 3r+1, 3r+2) of one input tile; at 1 x 1 it is three input
// tiles.  Workgroup = (group; 128 output channels; token slice), 8 waves.
// Wave w owns input channels 32 (w & 3) .. +31 of the three units and output
// channels 64 (w >> 2) .. +63: 3 x 2 blocks of 32 x 32 (96 accumulators), so
// each dY fragment feeds three units.  An empty unit stages zeros and stores
// nothing.
//
// The contraction runs over tokens while both operands are stored with
// channels contiguous.  Each step of 64 tokens is staged as it is stored:
// the gathered X rows of the three units (through N[k][unit's tap]) and the
// dY rows, 128 channels each, go straight from memory into LDS through
// buffer_load ... lds (gfx950: 16 bytes per lane, 1 KB per wave instruction,
// no registers and no LDS store instructions).  The MFMA fragments, which
// need 8 tokens per lane along k, come from those rows through the
// transposing LDS read ds_read_b64_tr_b16.  Step s + 1 is requested into
// the free buffer during step s, after its second k-step of MFMAs; each step
// ends with a single barrier, which also waits for those loads.  Staging
// 8 x 8 blocks through registers with v_perm transposes and LDS stores took
// 8-13% longer per call.
//
// The N entries a step needs (64 tokens x 3 units) are fetched once per
// workgroup by one wave, lane = token, two steps ahead, and passed through a
// small double-buffered LDS table: per-thread loads would request each entry
// 16 times and touch 8 cache lines per instruction for 32 useful bytes.
//
// All global reads are raw buffer loads with 32-bit offsets: rows of pruned
// neighbours and tokens past the slice get an out-of-range offset and read
// as zeros without a memory request or a branch.  The host sends inputs
// larger than the buffer range (2 GiB) to the VALU kernel.
constexpr int DW_BI = 128, DW_BO = 128, DW_TK = 64, DW_THREADS = 512;
// A staged tile: the step's 64 rows of 128 channels (256 bytes), row-major.
// A direct load writes 4 rows (1 KB) per wave instruction; token T = 16 q + b
// (b = 0..15, q = 0..3) is row q of block b, blocks 1088 bytes apart, so
// that the four consecutive tokens of a transposing read start in four
// different 64-byte bank quarters.
constexpr int DW_BLK = 1088;                      // bytes per block of 4 rows
constexpr int DW_TILEB = 16 * DW_BLK;             // bytes per tile
constexpr int DW_BUFB = 4 * DW_TILEB;             // 3 X tiles + 1 dY tile
constexpr int DW_NTAB = 2 * 3 * DW_TK;            // N table: [2 buffers][3 units][64 tokens]

typedef short v4s_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s_t lds_v4s_t;
__device__ __forceinline__ v4s_t tr_read(const char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t*)(p));
}
__device__ __forceinline__ bf16x8_t cat8(v4s_t lo, v4s_t hi) {
    const short8_t v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8_t, v);
}
__device__ __forceinline__ int tok_addr(int T) { return (T & 15) * DW_BLK + (T >> 4) * 256; }

__global__ __launch_bounds__(DW_THREADS) void k_dw_mfma(const uint16_t* __restrict__ X,
                                                        const int32_t* __restrict__ Nt,
                                                        const uint16_t* __restrict__ dY,
                                                        float* __restrict__ out, float* __restrict__ dbout,
                                                        int n, int Ci, int Co, int taps, int slice_tokens,
                                                        int direct, int accumulate) {
    // Two buffers as two arrays: the compiler then sees that a step's direct
    // loads (into one) never alias its fragment reads (from the other) and
    // waits for them only at the barrier.
    __shared__ __align__(16) char sbuf0[DW_BUFB];
    __shared__ __align__(16) char sbuf1[DW_BUFB];
    __shared__ int ntab[DW_NTAB];

    // 1-D grid of tiles x slices: logical id = slice * tiles + tile, so the
    // tiles of one token slice (which gather the same X and dY rows) sit
    // together on one XCD and share its L2.
    const int units = taps * (Ci / DW_BI);
    const int groups = (units + 2) / 3;
    const int tiles = groups * (Co / DW_BO);
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int slice = logical / tiles;
    const int bid = logical % tiles;
    const int grp = bid % groups;
    const int o0 = (bid / groups) * DW_BO;
    const int kbeg = slice * slice_tokens;
    const int cnt = max(0, min(n - kbeg, slice_tokens));
    const int steps = (cnt + DW_TK - 1) / DW_TK;
    // db: the 16 eight-channel chunks of the tile's 128 output channels are
    // dealt out over the groups (chunk c to group c mod groups), and within
    // a workgroup chunk number w of its own to wave w, lane = token (with one
    // group, a second chunk w + 8).  Summing all of db in one group made its
    // two workgroups per slice the last to finish.
    const int nch_db = dbout != nullptr ? (16 - grp + groups - 1) / groups : 0;   // chunks of this group

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wi = wave & 3, wo = wave >> 2;
    // staging role: tile (wave >> 1: units 0..2, then dY), blocks 8 (wave & 1) .. +7
    const int tile = wave >> 1;
    const bool is_x = tile < 3;
    const int unit = 3 * grp + (is_x ? tile : 0);
    const bool xlive = is_x && unit < units;
    const int ui0 = (unit / taps) * DW_BI;
    const uint32_t nrow = static_cast<uint32_t>(taps) * 4;
    const rsrc_t rX = make_rsrc(X, static_cast<uint32_t>(n) * Ci * 2);
    const rsrc_t rN = make_rsrc(Nt + static_cast<int64_t>(kbeg) * taps, static_cast<uint32_t>(cnt) * nrow);
    const rsrc_t rY = make_rsrc(dY + static_cast<int64_t>(kbeg) * Co, static_cast<uint32_t>(cnt) * Co * 2);
    // lane of a direct load: row q = lane >> 4 of the block, 16-byte chunk lane & 15
    const int dq = lane >> 4, dch = lane & 15;
    const uint32_t xCol = (ui0 + dch * 8) * 2, rowX = Ci * 2, rowY = Co * 2;
    const uint32_t yCol = (o0 + dch * 8) * 2;
    const int blk0 = (wave & 1) * 8;

    // N entries: the loader wave (lane = token) fetches the three units'
    // columns two steps ahead into a double-buffered table.
    const bool loader = wave == 6;
    int nreg[3], ltap[3];
#pragma unroll
    for (int t = 0; t < 3; ++t) ltap[t] = 3 * grp + t < units ? (3 * grp + t) % taps : -1;
    auto fetch_n = [&](int s) {
        const uint32_t base = static_cast<uint32_t>(s * DW_TK + lane) * nrow;
#pragma unroll
        for (int t = 0; t < 3; ++t) nreg[t] = ltap[t] >= 0 ? load4(rN, base + ltap[t] * 4) : -1;
    };
    auto put_n = [&](int s) {
#pragma unroll
        for (int t = 0; t < 3; ++t) ntab[((s & 1) * 3 + t) * DW_TK + lane] = nreg[t];
    };
    typedef __attribute__((address_space(3))) void lds_void_t;
    // Stage step s into `buf`: 8 direct loads per wave, block blk0 + j
    // holding tokens 16 q + blk0 + j.  Rows of pruned neighbours, of empty
    // units and of tokens past the slice read as zeros.
    // this lane's 8 table entries of step s (tokens 16 dq + blk0 .. +7), two 16-byte reads
    auto entries = [&](int s, int4& e0, int4& e1) {
        const int* nt = &ntab[((s & 1) * 3 + (is_x ? tile : 0)) * DW_TK + 16 * dq + blk0];
        e0 = *reinterpret_cast<const int4*>(nt);
        e1 = *reinterpret_cast<const int4*>(nt + 4);
    };
    auto issue = [&](int s, char* buf, const int4& e0, const int4& e1) {
        char* tb = buf + tile * DW_TILEB;
        const int lim = cnt - s * DW_TK;
        const int m8[8] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y, e1.z, e1.w};
        const rsrc_t rs = is_x ? rX : rY;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int T = 16 * dq + blk0 + j;
            const int m = m8[j];
            const uint32_t xo = (xlive && T < lim && static_cast<unsigned>(m) < static_cast<unsigned>(n))
                                    ? __umul24(static_cast<unsigned>(m), rowX) + xCol : kOob;
            const uint32_t yo = T < lim ? static_cast<uint32_t>(s * DW_TK + T) * rowY + yCol : kOob;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(tb + (blk0 + j) * DW_BLK), 16,
                                                     is_x ? xo : yo, 0, 0, 0);
        }
    };

    // Fragment reads through ds_read_b64_tr_b16.  Source lane: G = lane >> 4,
    // a = lane & 3, v = (lane >> 2) & 3, k half kh = G >> 1; it names the
    // 8-byte piece of token 32 kh + 8 ks + 4 h + v at channel 16 (G & 1) + 4 a
    // of the wave's 32 (A) or 32-of-64 (B) channels.  The read returns to
    // lane l channel l mod 32 of four consecutive tokens, so two reads (h =
    // 0, 1) give the 8 tokens of the lane's k slots; A and B use the same
    // token order, so every product meets its partner.
    const int G = lane >> 4, fa = lane & 3, fv = (lane >> 2) & 3, kh = G >> 1;
    const int colA = (wi * 32 + 16 * (G & 1) + 4 * fa) * 2;
    const int colB = (wo * 64 + 16 * (G & 1) + 4 * fa) * 2;

    floatx16_t acc[3][2];
#pragma unroll
    for (int t = 0; t < 3; ++t)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[t][b] = zero16();
    // db: thread = (16-byte chunk tid & 15 of the 128 output channels,
    // tokens tid >> 4 and 32 + (tid >> 4))
    const int wv = tid >> 6;                  // the wave, as a lane value (for the db chunk tests)
    const bool db0 = wv < nch_db, db1 = wv + 8 < nch_db;
    const int dbc0 = grp + wv * groups, dbc1 = grp + (wv + 8) * groups;     // chunk indices (when live)
    float dbacc[2][8];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) dbacc[u][e] = 0.f;

    auto stage = [&](int s, char* buf) {
        int4 e0, e1;
        entries(s, e0, e1);
        issue(s, buf, e0, e1);
    };
    // Step s's MFMAs from buffer xb.  With `more`, step s + 1 is staged into
    // nxt: its table entries are read first and its direct loads issued
    // after the second k-step, so that neither the table read's latency nor
    // the issue of the loads comes before the first MFMAs (issued at the
    // start of the step, they cost 9-12% of the call), while the loads still
    // have two k-steps to land before the barrier.
    auto mma_step = [&](const char* xb, int s, char* nxt, auto more_c) {
        constexpr bool more = decltype(more_c)::value;
        const char* yb = xb + 3 * DW_TILEB;
        int4 e0, e1;
        if constexpr (more) entries(s + 1, e0, e1);
        // k-step ks's fragments are read during k-step ks - 1: after the
        // barrier every wave of the workgroup starts a step at once, and
        // reading a k-step's fragments just before its own MFMAs had all of
        // them reading (MFMAs idle) and then all multiplying (LDS idle).
        // Scheduling barriers keep each k-step's reads ahead of the MFMAs of
        // the previous one.
        auto frags = [&](int ks, bf16x8_t* a, bf16x8_t* b) __attribute__((always_inline)) {
            const int t0 = 32 * kh + 8 * ks + fv;
            const int r0 = tok_addr(t0), r1 = tok_addr(t0 + 4);
#pragma unroll
            for (int t = 0; t < 3; ++t)
                a[t] = cat8(tr_read(xb + t * DW_TILEB + r0 + colA), tr_read(xb + t * DW_TILEB + r1 + colA));
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
                b[nb] = cat8(tr_read(yb + r0 + colB + nb * 64), tr_read(yb + r1 + colB + nb * 64));
        };
        bf16x8_t a[3], b[2], an[3], bn[2];
        frags(0, a, b);
#pragma unroll
        for (int ks = 0; ks < DW_TK / 16; ++ks) {
            if (ks < DW_TK / 16 - 1) frags(ks + 1, an, bn);
            if constexpr (more) {
                if (ks == 2) issue(s + 1, nxt, e0, e1);
            }
#pragma unroll
            for (int t = 0; t < 3; ++t)
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) acc[t][nb] = mfma32(a[t], b[nb], acc[t][nb]);
            // Two of the next k-step's reads after each MFMA: in-order issue
            // would otherwise hold all ten reads behind the six MFMAs' issue.
            if (ks < DW_TK / 16 - 1) {
                const bool dma = more && ks == 2;
                if (dma) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x020, 8, 0);
                }
#pragma unroll
                for (int i = 0; i < 5; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                }
                if (!dma) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int t = 0; t < 3; ++t) a[t] = an[t];
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) b[nb] = bn[nb];
        }
        if (db0) {
            // this lane's token of the step; tokens past the slice were
            // staged as zeros
            auto add8 = [&](int c, float* acc8) __attribute__((always_inline)) {
                const uint4 v = *reinterpret_cast<const uint4*>(yb + tok_addr(lane) + c * 16);
                const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    acc8[2 * h] += bf16_to_f32(static_cast<uint16_t>(w[h] & 0xffffu));
                    acc8[2 * h + 1] += bf16_to_f32(static_cast<uint16_t>(w[h] >> 16));
                }
            };
            add8(dbc0, dbacc[0]);
            if (db1) add8(dbc1, dbacc[1]);
        }
    };

    // prologue: table entries of steps 0 and 1, step 0 staged
    if (loader) {
        if (steps > 0) { fetch_n(0); put_n(0); }
        if (steps > 1) { fetch_n(1); put_n(1); }
        if (steps > 2) fetch_n(2);
    }
    __syncthreads();
    if (steps > 0) stage(0, sbuf0);
    __syncthreads();                       // also waits for the direct loads

    // Step s: step s + 1 is staged into the other buffer (last read in step
    // s - 1; its table entries were written in step s - 1), the loader puts
    // step s + 2's entries into the table slot of step s's (read in step
    // s - 1) and fetches step s + 3's; one barrier per step waits for all of
    // it, the direct loads included.
    // Whether a step stages the next one is a compile-time flag (only the
    // last step does not), so that each step is one straight-line block the
    // scheduler can interleave.
    auto step = [&](int s, const char* cur, char* nxt, auto more_c) {
        if (loader && s + 2 < steps) {
            put_n(s + 2);
            if (s + 3 < steps) fetch_n(s + 3);
        }
        mma_step(cur, s, nxt, more_c);
        __syncthreads();
    };
    using stage_next = std::integral_constant<bool, true>;
    using last_step = std::integral_constant<bool, false>;
    int s = 0;
    for (; s + 2 < steps; s += 2) {
        step(s, sbuf0, sbuf1, stage_next{});
        step(s + 1, sbuf1, sbuf0, stage_next{});
    }
    if (s + 1 < steps) {
        step(s, sbuf0, sbuf1, stage_next{});
        step(s + 1, sbuf1, sbuf0, last_step{});
    } else if (s < steps) {
        step(s, sbuf0, sbuf1, last_step{});
    }

    float* dst = out + (direct ? 0 : static_cast<int64_t>(slice) * taps * Ci * Co);
    const int l32 = lane & 31, lhi = lane >> 5;
#pragma unroll
    for (int t = 0; t < 3; ++t) {
        const int u = 3 * grp + t;
        if (u >= units) continue;
        const int i0 = (u / taps) * DW_BI;
        float* dj = dst + static_cast<int64_t>(u % taps) * Ci * Co;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int g = 0; g < 4; ++g)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int i = i0 + wi * 32 + g * 8 + lhi * 4 + q;
                    const int o = o0 + wo * 64 + nb * 32 + l32;
                    float* d = dj + static_cast<int64_t>(i) * Co + o;
                    const float v = acc[t][nb][g * 4 + q];
                    *d = (direct && accumulate) ? *d + v : v;
                }
    }
    if (nch_db > 0) {
        // each chunk's 64 lanes added in lane order, per channel
        float* red = reinterpret_cast<float*>(sbuf0);
        __syncthreads();
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e) red[(u * 8 + e) * DW_THREADS + tid] = dbacc[u][e];
        __syncthreads();
        // thread (u, chunk slot w, channel e) = tid: u = tid >> 6, w = (tid >> 3) & 7, e = tid & 7
        if (tid < 128) {
            const int u = tid >> 6, w = (tid >> 3) & 7, e = tid & 7;
            const int k = w + 8 * u;                         // the group's chunk number
            if (k < nch_db) {
                const int c = grp + k * groups;
                float v = 0.f;
                for (int l = 0; l < 64; ++l) v += red[(u * 8 + e) * DW_THREADS + w * 64 + l];
                float* d = dbout + (direct ? 0 : static_cast<int64_t>(slice) * Co) + o0 + c * 8 + e;
                *d = (direct && accumulate) ? *d + v : v;
            }
        }
    }
}

// db partials: block = 64 columns x 4 row phases; fixed-order combine in LDS.
// With one slice (`direct`) the sums go straight to db, added to it under
// `accumulate`.
template <typename T>
__global__ __launch_bounds__(256) void k_db_partial(const T* __restrict__ dY, float* __restrict__ part,
                                                    int n, int Co, int64_t slice_tokens, int direct,
                                                    int accumulate) {
    __shared__ float red[4][64];
    const int c = threadIdx.x & 63, ph = threadIdx.x >> 6;
    const int o = blockIdx.x * 64 + c;
    const int64_t kbeg = static_cast<int64_t>(blockIdx.y) * slice_tokens;
    const int64_t kend = min(static_cast<int64_t>(n), kbeg + slice_tokens);
    float sum = 0.f;
    if (o < Co)
        for (int64_t k = kbeg + ph; k < kend; k += 4) sum += Elem<T>::load(dY + k * Co + o);
    red[ph][c] = sum;
    __syncthreads();
    if (ph == 0 && o < Co) {
        const float v = ((red[0][c] + red[1][c]) + red[2][c]) + red[3][c];
        float* d = part + static_cast<int64_t>(blockIdx.y) * Co + o;
        *d = (direct && accumulate) ? *d + v : v;
    }
}

// out[e] (+)= sum_{s < slices} part[s][e], s ascending (4 floats per thread).
// The db partials ride along: block 0 also reduces them (Co floats, one per
// thread, same order), which saves a launch.
__global__ __launch_bounds__(256) void k_reduce_slices4(const float4* __restrict__ part, float4* __restrict__ out,
                                                        int64_t count4, int slices, int accumulate,
                                                        const float* __restrict__ dbpart, float* __restrict__ db,
                                                        int Co) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < count4; e += stride) {
        // loads issued 8 slices at a time (one wait per batch instead of one
        // per slice), added in slice order
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        int s = 0;
        for (; s + 8 <= slices; s += 8) {
            float4 p[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) p[u] = part[static_cast<int64_t>(s + u) * count4 + e];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                v.x += p[u].x; v.y += p[u].y; v.z += p[u].z; v.w += p[u].w;
            }
        }
        for (; s < slices; ++s) {
            const float4 p = part[static_cast<int64_t>(s) * count4 + e];
            v.x += p.x; v.y += p.y; v.z += p.z; v.w += p.w;
        }
        if (accumulate) {
            const float4 o = out[e];
            v.x = o.x + v.x; v.y = o.y + v.y; v.z = o.z + v.z; v.w = o.w + v.w;
        }
        out[e] = v;
    }
    if (db && blockIdx.x == 0)
        for (int o = threadIdx.x; o < Co; o += blockDim.x) {
            // loads issued 8 at a time, added in slice order
            float v = 0.f;
            int s = 0;
            for (; s + 8 <= slices; s += 8) {
                float p[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) p[u] = dbpart[static_cast<int64_t>(s + u) * Co + o];
#pragma unroll
                for (int u = 0; u < 8; ++u) v += p[u];
            }
            for (; s < slices; ++s) v += dbpart[static_cast<int64_t>(s) * Co + o];
            db[o] = accumulate ? db[o] + v : v;
        }
}

// out[e] (+)= sum_{s < slices} part[s][e], s ascending.
__global__ __launch_bounds__(256) void k_reduce_slices(const float* __restrict__ part, float* __restrict__ out,
                                                       int64_t count, int slices, int accumulate) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < count; e += stride) {
        float v = 0.f;
        int s = 0;
        for (; s + 8 <= slices; s += 8) {
            float p[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) p[u] = part[static_cast<int64_t>(s + u) * count + e];
#pragma unroll
            for (int u = 0; u < 8; ++u) v += p[u];
        }
        for (; s < slices; ++s) v += part[static_cast<int64_t>(s) * count + e];
        out[e] = accumulate ? out[e] + v : v;
    }
}

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

constexpr int64_t kDwSlots = 192;   // workgroups per dispatch round in the cost model

DwPlan plan_dw(int64_t n, int Ci, int Co, bool bf16, int taps) {
    DwPlan p{};
    p.taps = taps;
    // The MFMA kernel addresses X, dY and N through 32-bit buffer offsets.
    p.mfma = bf16 && Ci % DW_BI == 0 && Co % DW_BO == 0 && n * Ci * 2 <= kMaxRange &&
             n * Co * 2 <= kMaxRange && n * taps * 4 <= kMaxRange;
    int64_t slices;
    const int64_t step = p.mfma ? DW_TK : 16;
    if (p.mfma) {
        // Split-K factor from a small cost model: one workgroup per compute
        // unit at ~4 TFLOP/s, counted in whole dispatch rounds of
        // kDwSlots workgroups, plus the fp32 partials written and read back
        // (~5 TB/s) and a fixed cost for the extra reduction launch.  The
        // rounds are counted against three quarters of a 256-CU part: in a
        // training step the weight gradient runs beside the input gradient,
        // and on the c5 backward the smaller split (16 slices instead of 21
        // at 58,822 tokens) made the whole step 2.5-3% faster although the
        // call alone is ~7% slower.  Depends on the arguments only, so
        // workspace sizing and the call agree.
        const int64_t tiles = ceil_div(static_cast<int64_t>(taps) * (Ci / DW_BI), 3) * (Co / DW_BO);
        const double flops = 2.0 * static_cast<double>(n) * static_cast<double>(3 * tiles / (Co / DW_BO)) * DW_BI * Co;
        const double dwb = static_cast<double>(taps) * Ci * Co * 4;
        double best = 1e30;
        slices = 1;
        for (int64_t s = 1; s <= 64; ++s) {
            if (s > 1 && ceil_div(n, s) < 4 * DW_TK) break;
            const double rounds = static_cast<double>(ceil_div(tiles * s, kDwSlots));
            const double t = rounds * flops / static_cast<double>(tiles * s) / 4e12 +
                             (s > 1 ? (2.0 * static_cast<double>(s) * dwb / 5e12 + 4e-6) : 0.0);
            if (t < best) { best = t; slices = s; }
        }
    } else {
        const int64_t tiles = static_cast<int64_t>(taps) * ceil_div(Ci, 64) * ceil_div(Co, 64);
        slices = ceil_div(512, tiles);
        slices = std::min<int64_t>(slices, std::max<int64_t>(1, n / 512));
        slices = std::max<int64_t>(1, std::min<int64_t>(slices, 64));
    }
    int64_t st = ceil_div(std::max<int64_t>(n, 1), slices);
    st = ceil_div(st, step) * step;
    slices = std::max<int64_t>(1, ceil_div(n, st));
    p.slices = static_cast<int>(slices);
    p.slice_tokens = st;
    p.partial_floats = slices > 1 ? static_cast<size_t>(slices) * taps * Ci * Co : 0;
    p.db_floats = static_cast<size_t>(slices) * Co;
    return p;
}

size_t dw_workspace_bytes(const DwPlan& p) {
    auto up = [](size_t b) { return (b + 255) & ~static_cast<size_t>(255); };
    return up(p.partial_floats * sizeof(float)) + up(p.db_floats * sizeof(float));
}

// Phase 1: the partial kernels (dW straight into dW with one slice, else
// the slices' partials into the workspace; db partials likewise).
hipError_t launch_dw_partials(const DwPlan& plan, bool bf16, const void* X, const int32_t* N, const void* dY,
                              float* dW, float* db, int64_t n, int Ci, int Co, int accumulate, void* ws,
                              hipStream_t stream) {
    auto up = [](size_t b) { return (b + 255) & ~static_cast<size_t>(255); };
    float* part = static_cast<float*>(ws);
    float* dbpart = reinterpret_cast<float*>(static_cast<char*>(ws) + up(plan.partial_floats * sizeof(float)));
    const bool direct = plan.slices == 1;
    hipError_t err;
    if (plan.mfma) {
        const int groups = (plan.taps * (Ci / DW_BI) + 2) / 3;
        dim3 grid(groups * (Co / DW_BO) * plan.slices);
        hipLaunchKernelGGL(k_dw_mfma, grid, dim3(DW_THREADS), 0, stream, static_cast<const uint16_t*>(X), N,
                           static_cast<const uint16_t*>(dY), direct ? dW : part,
                           db ? (direct ? db : dbpart) : nullptr, static_cast<int>(n), Ci, Co, plan.taps,
                           static_cast<int>(plan.slice_tokens), direct ? 1 : 0, accumulate);
        return hipGetLastError();
    }
    err = launch_dw_valu(bf16, X, N, dY, direct ? dW : part, n, Ci, Co, plan.taps, plan.slices,
                         plan.slice_tokens, direct ? 1 : 0, accumulate, stream);
    if (err != hipSuccess || !db) return err;
    dim3 grid(static_cast<unsigned>(ceil_div(Co, 64)), plan.slices);
    float* dbdst = direct ? db : dbpart;
    if (bf16)
        hipLaunchKernelGGL(k_db_partial<uint16_t>, grid, dim3(256), 0, stream, static_cast<const uint16_t*>(dY),
                           dbdst, static_cast<int>(n), Co, plan.slice_tokens, direct ? 1 : 0, accumulate);
    else
        hipLaunchKernelGGL(k_db_partial<float>, grid, dim3(256), 0, stream, static_cast<const float*>(dY), dbdst,
                           static_cast<int>(n), Co, plan.slice_tokens, direct ? 1 : 0, accumulate);
    return hipGetLastError();
}

// Phase 2: the fixed-order reduction of whatever phase 1 left in the
// workspace (nothing with one slice on the MFMA path).
hipError_t launch_dw_reduce(const DwPlan& plan, float* dW, float* db, int Ci, int Co, int accumulate,
                            const void* ws, hipStream_t stream) {
    auto up = [](size_t b) { return (b + 255) & ~static_cast<size_t>(255); };
    const float* part = static_cast<const float*>(ws);
    const float* dbpart =
        reinterpret_cast<const float*>(static_cast<const char*>(ws) + up(plan.partial_floats * sizeof(float)));
    const bool direct = plan.slices == 1;
    hipError_t err = hipSuccess;
    // With one slice both kernels wrote db directly; otherwise the db
    // partials go through the dW reduction launch.
    bool db_done = db && direct;
    if (!direct) {
        const int64_t count = static_cast<int64_t>(plan.taps) * Ci * Co;
        if (count % 4 == 0) {
            const int blocks = static_cast<int>(std::min<int64_t>(ceil_div(count / 4, 256), 8192));
            hipLaunchKernelGGL(k_reduce_slices4, dim3(blocks), dim3(256), 0, stream,
                               reinterpret_cast<const float4*>(part), reinterpret_cast<float4*>(dW), count / 4,
                               plan.slices, accumulate, db ? dbpart : nullptr, db, Co);
            db_done = db != nullptr;
        } else {
            const int blocks = static_cast<int>(std::min<int64_t>(ceil_div(count, 256), 8192));
            hipLaunchKernelGGL(k_reduce_slices, dim3(blocks), dim3(256), 0, stream, part, dW, count,
                               plan.slices, accumulate);
        }
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if (db && !db_done) {
        const int blocks = static_cast<int>(ceil_div(Co, 256));
        hipLaunchKernelGGL(k_reduce_slices, dim3(blocks), dim3(256), 0, stream, dbpart, db,
                           static_cast<int64_t>(Co), plan.slices, accumulate);
        err = hipGetLastError();
    }
    return err;
}

hipError_t launch_dw(const DwPlan& plan, bool bf16, const void* X, const int32_t* N, const void* dY,
                     float* dW, float* db, int64_t n, int Ci, int Co, int accumulate, void* ws,
                     hipStream_t stream) {
    hipError_t err = launch_dw_partials(plan, bf16, X, N, dY, dW, db, n, Ci, Co, accumulate, ws, stream);
    if (err != hipSuccess) return err;
    return launch_dw_reduce(plan, dW, db, Ci, Co, accumulate, ws, stream);
}

}  // namespace svc
