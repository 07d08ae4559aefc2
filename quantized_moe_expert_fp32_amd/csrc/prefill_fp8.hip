// FP8 route of the prompt experts: the experts upcast once to FP8 so the prompt's
// grouped GEMMs run on the FP8 matrix cores ("R9700: the 35B only one runtime could
// load", R9700 vLLM blog part 13, its closing list of kernel work; there aimed at
// RDNA4's FP8 WMMA, here at CDNA4's v_mfma_scale_f32_16x16x128_f8f6f4).
//
// Numbers (OCP FP8 E4M3, round to nearest even, by v_cvt_pk_fp8_f32):
//   * each weight row is formed as w = fma(scale, q, bias) in fp32 and stored as
//     codes of w * 2^-e with e = floor(log2 max|w|) - 7 (the row's largest
//     magnitude maps into [128, 256): no code saturates), the row scale 2^e kept as
//     one float;
//   * the activation rows entering each projection (x for gate/up, the bf16 SwiGLU
//     intermediate h for down) are quantised the same way, one 2^e per row;
//   * a projection is acc * 2^e_row * 2^e_col with acc the fp32 MFMA sum of code
//     products (each exact in fp32). Every output's arithmetic depends on its own
//     activation row and weight row only, as in the exact path.
// The route reuses the exact path's routing, dispatch (tiles of 128 rows) and
// combine; h stays bf16 between the two GEMMs, as there.
//
// Tiles: up to 128 expert-sorted rows x 256 weight rows per workgroup of four
// wavefronts (gate/up: 128 gate rows and the matching 128 up rows; down: 256
// output columns), on v_mfma_scale_f32_32x32x64_f8f6f4. Wavefront w owns two
// 32-row blocks of the weight rows over every tile row, so each fragment read from
// LDS feeds two (B) or up to four (A) products, and a wavefront holds a gate row
// block and its up row block side by side.
#include "mfma_common.h"
#include "moe_internal.h"
#include "prefill_internal.h"

namespace moe {

// ---------------------------------------------------------------- FP8 expert buffer
// Per expert (stride bytes): gate codes [I][Hp] | up codes [I][Hp] | down codes
// [H][Ip] | row scales float [2I + H] (gate rows, up rows, down rows). Rows are
// padded with zero codes to Hp = H and Ip = I rounded up to 128 (one MFMA depth).
struct Fp8Layout {
    size_t up, down, scales, stride;
    int Hp, Ip;
};

static Fp8Layout fp8_layout(const moe_shape& s) {
    Fp8Layout L;
    L.Hp = (int)align_up((size_t)s.hidden, 128);
    L.Ip = (int)align_up((size_t)s.inter, 128);
    L.up = (size_t)s.inter * L.Hp;
    L.down = 2 * L.up;
    L.scales = L.down + (size_t)s.hidden * L.Ip;
    L.stride = align_up(L.scales + 4 * (size_t)(2 * s.inter + s.hidden), 256);
    return L;
}

// e = floor(log2 amax) - 7 (v_frexp_exp gives amax = f 2^x, f in [0.5, 1)); 0 for a zero row.
__device__ __forceinline__ int fp8_row_exp(float amax) {
    return amax > 0.f ? __builtin_amdgcn_frexp_expf(amax) - 1 - 7 : 0;
}

// Four floats (|v| < 256) as four E4M3 codes, value j in byte j.
__device__ __forceinline__ uint32_t fp8x4(float a, float b, float c, float d) {
    uint32_t r = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, (int)r, true);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

// ---------------------------------------------------------------- packing
// One wavefront per weight row; row r of expert m in the order gate 0..I-1, up
// 0..I-1, down 0..H-1. Lane l forms the weights 8l + 512j .. +8 (two passes over the
// canonical row: the row's max, then the codes).
template <int BITS>
__global__ __launch_bounds__(256) void pack_fp8_kernel(moe_expert_canon c, int H, int I, int M, Fp8Layout L,
                                                       uint8_t* __restrict__ out) {
    const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int R = 2 * I + H;
    if (row >= (long long)M * R) return;
    const int m = (int)(row / R), r = (int)(row % R);
    const uint8_t* q;
    const uint16_t *sc, *bi;
    int K, Kp;
    uint8_t* dst = out + (size_t)m * L.stride;
    if (r < 2 * I) {
        const int i = r < I ? r : r - I;
        const size_t rr = (size_t)m * I + i;
        K = H;
        Kp = L.Hp;
        q = (r < I ? c.q_gate : c.q_up) + rr * (size_t)(H * BITS / 8);
        sc = (r < I ? c.s_gate : c.s_up) + rr * (size_t)(H / 64);
        bi = (r < I ? c.b_gate : c.b_up) + rr * (size_t)(H / 64);
        dst += (r < I ? 0 : L.up) + (size_t)i * L.Hp;
    } else {
        const int n = r - 2 * I;
        const size_t rr = (size_t)m * H + n;
        K = I;
        Kp = L.Ip;
        q = c.q_down + rr * (size_t)(I * BITS / 8);
        sc = c.s_down + rr * (size_t)(I / 64);
        bi = c.b_down + rr * (size_t)(I / 64);
        dst += L.down + (size_t)n * L.Ip;
    }
    auto weights = [&](int c0, float w[8]) {
        const float s = bf16_to_f32(sc[c0 / 64]), b = bf16_to_f32(bi[c0 / 64]);
        uint32_t qv[8];
        if constexpr (BITS == 4) {
            const uint32_t d = *reinterpret_cast<const uint32_t*>(q + c0 / 2);  // element 2j: low nibble of byte j
#pragma unroll
            for (int j = 0; j < 8; ++j) qv[j] = (d >> (4 * j)) & 15u;
        } else {
            const uint2 d = *reinterpret_cast<const uint2*>(q + c0);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                qv[j] = (d.x >> (8 * j)) & 255u;
                qv[4 + j] = (d.y >> (8 * j)) & 255u;
            }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) w[j] = fmaf(s, (float)qv[j], b);
    };
    float amax = 0.f;
    for (int c0 = 8 * lane; c0 < K; c0 += 512) {
        float w[8];
        weights(c0, w);
#pragma unroll
        for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(w[j]));
    }
    const int e = fp8_row_exp(wave_max(amax));
    for (int c0 = 8 * lane; c0 < Kp; c0 += 512) {
        uint2 code = make_uint2(0u, 0u);
        if (c0 < K) {
            float w[8];
            weights(c0, w);
            code.x = fp8x4(ldexpf(w[0], -e), ldexpf(w[1], -e), ldexpf(w[2], -e), ldexpf(w[3], -e));
            code.y = fp8x4(ldexpf(w[4], -e), ldexpf(w[5], -e), ldexpf(w[6], -e), ldexpf(w[7], -e));
        }
        *reinterpret_cast<uint2*>(dst + c0) = code;
    }
    if (lane == 0)
        reinterpret_cast<float*>(out + (size_t)m * L.stride + L.scales)[r] = ldexpf(1.f, e);
}

// ---------------------------------------------------------------- activation rows
// One wavefront per bf16 row src [rows][K] -> codes dst [rows][Kp] (zero padded) and
// scale[row] = 2^e. With live != nullptr only rows below *live are quantised.
__global__ __launch_bounds__(256) void quant_rows_fp8_kernel(const uint16_t* __restrict__ src, long long rows,
                                                             const int32_t* __restrict__ live, int K, int Kp,
                                                             uint8_t* __restrict__ dst, float* __restrict__ scale) {
    const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows || (live && row >= *live)) return;
    const uint16_t* sr = src + (size_t)row * K;
    float amax = 0.f;
    for (int c0 = 8 * lane; c0 < K; c0 += 512) {
        const uint4 v = *reinterpret_cast<const uint4*>(sr + c0);
        const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j)
            amax = fmaxf(amax, fmaxf(fabsf(bf16_to_f32(d[j] & 0xFFFFu)), fabsf(bf16_to_f32(d[j] >> 16))));
    }
    const int e = fp8_row_exp(wave_max(amax));
    uint8_t* dr = dst + (size_t)row * Kp;
    for (int c0 = 8 * lane; c0 < Kp; c0 += 512) {
        uint2 code = make_uint2(0u, 0u);
        if (c0 < K) {
            const uint4 v = *reinterpret_cast<const uint4*>(sr + c0);
            auto f = [&](uint32_t d, int hi) { return ldexpf(bf16_to_f32(hi ? d >> 16 : d & 0xFFFFu), -e); };
            code.x = fp8x4(f(v.x, 0), f(v.x, 1), f(v.y, 0), f(v.y, 1));
            code.y = fp8x4(f(v.z, 0), f(v.z, 1), f(v.w, 0), f(v.w, 1));
        }
        *reinterpret_cast<uint2*>(dr + c0) = code;
    }
    if (lane == 0) scale[row] = ldexpf(1.f, e);
}

// ---------------------------------------------------------------- grouped FP8 GEMM
// A workgroup multiplies one tile (up to 128 expert-sorted rows) by NB8 = 256
// weight rows of the tile's expert over the whole K, in chunks of KC8 = 64 codes
// (one depth of v_mfma_scale_f32_32x32x64_f8f6f4). Per chunk, direct
// global-to-LDS loads stage the tile's rows x 64 B and the 256 weight rows x 64 B
// into a ring of three LDS stages that runs two chunks ahead of the one being
// multiplied. The ring (72 KiB) lets two workgroups share a CU, so one's prologue
// and epilogue overlap the other's main loop.
constexpr int BM8 = 128;
constexpr int NB8 = 256;
constexpr int KC8 = 64;
constexpr int B8_BYTES = NB8 * KC8;                 // 16 KiB
constexpr int RING8 = 3 * (BM8 * KC8 + B8_BYTES);  // 72 KiB: three stages of a full tile

struct Fp8GemmArgs {
    const uint8_t* w8;  // FP8 expert buffer
    Fp8Layout L;
    int H, I, S;
    const uint8_t* a8;     // gate/up: x codes [T][Hp]; down: h codes [T*S][Ip] (expert-sorted rows)
    const float* ascale;   // 2^e of each of those rows
    const int32_t* ntiles;
    const Tile* tiles;
    const int32_t* order;
    uint16_t* hbuf;        // gate/up output: h [T*S][I] bf16, expert-sorted rows
    float* y;              // down output: [T][S][H]
};

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// D += A B over one 32 x 32 x 64 block: lane l holds row (A) / column (B) l % 32,
// the 32 codes of k half l / 32 (16 from each uint4), and receives D[8 (r / 4) +
// 4 (l / 32) + r % 4][l % 32] in register r. Both operand scales are 2^0.
__device__ __forceinline__ f32x16_t mfma_fp8(const uint4& a0, const uint4& a1, const uint4& b0, const uint4& b1,
                                             const f32x16_t& c) {
    const i32x8_t a = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
    const i32x8_t b = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// 16-byte piece p of staged row r sits at position p ^ ((r >> 2) & 3) of the row's
// 64 bytes: the rows sharing a bank window read different pieces.
__device__ __forceinline__ int piece_pos(int r, int p) { return p ^ ((r >> 2) & 3); }

// GATEUP: weight rows 0..127 are gate rows cb*128 .., rows 128..255 the matching up
// rows; the epilogue writes h = bf16(silu(gate) * up). Else (down): weight rows are
// down rows cb*256 ..; the epilogue writes y[t][s][n] for the row's pick p = order[row].
// Wavefront w owns the weight rows n0(cs) .. +32, cs < 2 (gate/up: gate rows 32w ..
// and up rows 128 + 32w .., the same intermediate columns; down: rows 64w + 32cs ..)
// over all tile rows.
template <bool GATEUP>
__global__ __launch_bounds__(256, 2) void fp8_gemm_kernel(Fp8GemmArgs a) {
    constexpr int NCS = 2;
    extern __shared__ __attribute__((aligned(16))) uint8_t ring[];
    __shared__ uint32_t arow_lds[BM8];  // byte offset of each tile row in its source, ~0 beyond the tile
    __shared__ int32_t pick_lds[BM8];   // down: pick p = order[row] of each tile row
    __shared__ float as_lds[BM8];       // the tile rows' scales
    __shared__ float ws_lds[NB8];       // the weight rows' scales
    const int H = a.H, I = a.I, S = a.S;
    const int Kp = GATEUP ? a.L.Hp : a.L.Ip;  // codes per row of both operands
    const int nblk = GATEUP ? (I + 127) / 128 : (H + NB8 - 1) / NB8;
    int ti, cb;
    if (!xcd_item(*a.ntiles, nblk, ti, cb)) return;
    const Tile tl = a.tiles[ti];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, kh = lane >> 5;
    const int n_ms = (tl.nrows + 31) >> 5;
    const uint8_t* ebase = a.w8 + (size_t)tl.expert * a.L.stride;
    // weight row r of the workgroup: its byte offset in the expert and its scale's
    // index; rows beyond the matrix read row 0 and are never stored
    auto wrow = [&](int r, int& sidx) -> uint32_t {
        if constexpr (GATEUP) {
            const int i0 = cb * 128 + (r & 127), i = i0 < I ? i0 : 0;
            sidx = (r < 128 ? 0 : I) + i;
            return (uint32_t)((r < 128 ? 0 : a.L.up) + (size_t)i * Kp);
        } else {
            const int n0 = cb * NB8 + r, n = n0 < H ? n0 : 0;
            sidx = 2 * I + n;
            return (uint32_t)(a.L.down + (size_t)n * Kp);
        }
    };
    auto n0 = [&](int cs) -> int { return GATEUP ? cs * 128 + 32 * wave : 64 * wave + 32 * cs; };
    if (tid < BM8) {
        uint32_t off = 0xFFFFFFFFu;
        float sc = 0.f;
        int pick = 0;
        if (tid < tl.nrows) {
            const int p = a.order[tl.row0 + tid];
            const int src = GATEUP ? p / S : tl.row0 + tid;
            off = (uint32_t)src * (uint32_t)Kp;
            sc = a.ascale[src];
            pick = p;
        }
        arow_lds[tid] = off;
        as_lds[tid] = sc;
        pick_lds[tid] = pick;
    }
    {
        int sidx;
        wrow(tid, sidx);
        ws_lds[tid] = reinterpret_cast<const float*>(ebase + a.L.scales)[sidx];
    }
    __syncthreads();

    // ---- stage layout: A: the loaded rows x 64 B, then B: 256 rows x 64 B. One
    // load instruction covers 16 rows; lane l loads piece piece_pos(r, l & 3) of row
    // r = 16 i + (l >> 2) into position l & 3. Rows beyond the tile load row 0 of the
    // tile instead, so every lane issues every load and the wait for a chunk is an
    // exact vector-memory count.
    const uint32_t ring_lds = lds_addr(ring);
    uint32_t b_off[4];  // B: instruction 4 wave + i covers rows 16 (4 wave + i) .. +16
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 16 * (4 * wave + i) + (lane >> 2);
        int sidx;
        b_off[i] = wrow(r, sidx) + 16 * piece_pos(r, lane & 3);
    }

    f32x16_t acc[4][NCS];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int cs = 0; cs < NCS; ++cs)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[m][cs][r] = 0.f;
    // The K loop is instantiated for 1, 2 and 4 row blocks of 32 (the tile's count
    // rounded up), so its body is straight-line code.
    auto kloop = [&](auto nm_tag) __attribute__((always_inline)) {
        constexpr int NM = decltype(nm_tag)::value;
        constexpr int NA = NM >= 2 ? NM / 2 : 1;  // A instructions (16 rows each) per wavefront
        constexpr int LPC = NA + 4;               // loads per wavefront and chunk
        constexpr int SA = 4 * NA * 1024;         // A bytes per stage (64 NA rows)
        constexpr int STAGE = SA + B8_BYTES;
        constexpr int NS = RING8 / STAGE;         // stages
        static_assert(NS >= 3 && NS * STAGE <= RING8 && LPC * (NS - 2) < 64, "ring");
        const uint32_t arow0 = arow_lds[0];
        uint32_t a_off[NA];
#pragma unroll
        for (int i = 0; i < NA; ++i) {
            const int row = 16 * (NA * wave + i) + (lane >> 2);
            const uint32_t off = row < BM8 ? arow_lds[row] : 0xFFFFFFFFu;
            a_off[i] = (off == 0xFFFFFFFFu ? arow0 : off) + 16 * piece_pos(row, lane & 3);
        }
        auto issue = [&](int c) __attribute__((always_inline)) {
            const uint32_t st = ring_lds + (uint32_t)((c % NS) * STAGE);
            const uint8_t* ab = a.a8 + (size_t)c * KC8;
#pragma unroll
            for (int i = 0; i < NA; ++i) lds_dma16(ab, a_off[i], st + (NA * wave + i) * 1024);
            const uint8_t* bb = ebase + (size_t)c * KC8;
#pragma unroll
            for (int i = 0; i < 4; ++i) lds_dma16(bb, b_off[i], st + SA + (4 * wave + i) * 1024);
        };
        auto compute = [&](int c) __attribute__((always_inline)) {
            const uint8_t* st = ring + (size_t)(c % NS) * STAGE;
            uint4 b0[NCS], b1[NCS];
#pragma unroll
            for (int cs = 0; cs < NCS; ++cs) {
                const int n = n0(cs) + l32;
                const uint8_t* bp = st + SA + n * 64;
                b0[cs] = *reinterpret_cast<const uint4*>(bp + 16 * piece_pos(n, 2 * kh));
                b1[cs] = *reinterpret_cast<const uint4*>(bp + 16 * piece_pos(n, 2 * kh + 1));
            }
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                const int row = 32 * m + l32;
                const uint8_t* ar = st + row * 64;
                const uint4 a0 = *reinterpret_cast<const uint4*>(ar + 16 * piece_pos(row, 2 * kh));
                const uint4 a1 = *reinterpret_cast<const uint4*>(ar + 16 * piece_pos(row, 2 * kh + 1));
#pragma unroll
                for (int cs = 0; cs < NCS; ++cs) acc[m][cs] = mfma_fp8(a0, a1, b0[cs], b1[cs], acc[m][cs]);
            }
        };
        const int NC = Kp / KC8;
        for (int c = 0; c < NS - 1 && c < NC; ++c) issue(c);
        for (int c = 0; c < NC; ++c) {
            // this wavefront's loads of chunk c are done once only the later chunks'
            // (at most NS - 2 of them) are left
            wait_chunks<LPC, NS - 2>(NC - 1 - c);
            // every wavefront's loads of chunk c are in LDS, and every wavefront has
            // finished chunk c-1, whose stage the next loads refill
            lds_barrier();
            if (c + NS - 1 < NC) issue(c + NS - 1);
            compute(c);
        }
    };
    if (n_ms <= 1) kloop(std::integral_constant<int, 1>{});
    else if (n_ms <= 2) kloop(std::integral_constant<int, 2>{});
    else kloop(std::integral_constant<int, 4>{});

    // ---- epilogue: the ring's memory is free once every wavefront is past its last chunk
    __syncthreads();
    if constexpr (GATEUP) {
        // h = bf16(silu(g) * u) for intermediate columns i = cb*128 + c, c = 32 wave +
        // l32, staged as a bf16 tile in LDS, then stored with 16-byte row pieces.
        constexpr int HS = 128 + 8;  // tile row stride (bf16)
        uint16_t* hl = reinterpret_cast<uint16_t*>(ring);
        const int c = 32 * wave + l32;
        const float sg = ws_lds[c], su = ws_lds[128 + c];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            if (m < n_ms) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = 32 * m + 8 * (r >> 2) + 4 * kh + (r & 3);
                    const float gv = acc[m][0][r] * as_lds[row] * sg, uv = acc[m][1][r] * as_lds[row] * su;
                    // silu(g) = g / (1 + e^-g), e^-g = 2^(-g log2 e)
                    const float sl = gv * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-gv * 1.44269504088896341f));
                    hl[row * HS + c] = __builtin_bit_cast(uint16_t, (__bf16)(sl * uv));
                }
            }
        }
        __syncthreads();
        for (int it = 0; it < 8; ++it) {
            const int row = 16 * it + (tid >> 4), pc = tid & 15;
            if (row < tl.nrows && cb * 128 + 8 * pc < I)
                *reinterpret_cast<uint4*>(a.hbuf + (size_t)(tl.row0 + row) * I + cb * 128 + 8 * pc) =
                    *reinterpret_cast<const uint4*>(hl + row * HS + 8 * pc);
        }
    } else {
        // y[order[row]][cb*256 + n], staged 64 rows at a time as an fp32 tile in LDS
        // and stored with 16-byte row pieces, non-temporal (y is read once, by the
        // combine).
        constexpr int YS = NB8 + 4;  // tile row stride (floats)
        static_assert(64 * YS * 4 <= RING8, "y tile");
        float* yl = reinterpret_cast<float*>(ring);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            if (64 * half < tl.nrows) {
                if (half) __syncthreads();
#pragma unroll
                for (int mm = 0; mm < 2; ++mm) {
                    const int m = 2 * half + mm;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int rl = 32 * mm + 8 * (r >> 2) + 4 * kh + (r & 3);
                        const float sa = as_lds[64 * half + rl];
#pragma unroll
                        for (int cs = 0; cs < NCS; ++cs) {
                            const int n = n0(cs) + l32;
                            yl[rl * YS + n] = acc[m][cs][r] * sa * ws_lds[n];
                        }
                    }
                }
                __syncthreads();
                for (int it = 0; it < 16; ++it) {
                    const int rl = 4 * it + (tid >> 6), row = 64 * half + rl, pc = tid & 63;
                    if (row < tl.nrows && cb * NB8 + 4 * pc < H)
                        __builtin_nontemporal_store(*reinterpret_cast<const f32x4_t*>(yl + rl * YS + 4 * pc),
                                                    reinterpret_cast<f32x4_t*>(a.y + (size_t)pick_lds[row] * H +
                                                                               cb * NB8 + 4 * pc));
                }
            }
        }
    }
}

// Workspace of moe_experts_prefill_fp8: the dispatch (tiles of BM8 rows), x codes
// and scales, h, h codes and scales.
struct Fp8Ws {
    DispatchWs D;
    size_t x8, xs, h, h8, hs, total;
};

static Fp8Ws fp8_ws_layout(const moe_shape& s, int T) {
    Fp8Ws w;
    const Fp8Layout L = fp8_layout(s);
    const size_t P = (size_t)T * n_slots(s);
    size_t o = 0;
    w.D = dispatch_ws_layout(s, T, BM8, o);
    w.x8 = o; o = align_up(o + (size_t)T * L.Hp, 256);
    w.xs = o; o = align_up(o + 4 * (size_t)T, 256);
    w.h = o;  o = align_up(o + 2 * P * s.inter, 256);
    w.h8 = o; o = align_up(o + P * L.Ip, 256);
    w.hs = o; o = align_up(o + 4 * P, 256);
    w.total = o;
    return w;
}

}  // namespace moe

using namespace moe;

extern "C" size_t moe_experts_fp8_bytes(const moe_shape* shape) {
    if (validate_shape(shape) != MOE_OK) return 0;
    return fp8_layout(*shape).stride * (size_t)n_mats(*shape);
}

extern "C" moe_status moe_pack_experts_fp8(const moe_shape* shape, const moe_expert_canon* src_host, void* fp8,
                                           size_t fp8_bytes, void* stream) {
    clear_error();
    moe_status st = validate_shape(shape);
    if (st != MOE_OK) return st;
    const moe_shape& sh = *shape;
    if (!src_host || !fp8 || ((uintptr_t)fp8 & 255u))
        return fail(MOE_ERR_INVALID_ARG, "NULL source or FP8 buffer not 256-byte aligned");
    const moe_expert_canon& c = *src_host;
    if (!c.q_gate || !c.s_gate || !c.b_gate || !c.q_up || !c.s_up || !c.b_up || !c.q_down || !c.s_down || !c.b_down)
        return fail(MOE_ERR_INVALID_ARG, "NULL canonical array");
    if (((uintptr_t)c.q_gate | (uintptr_t)c.q_up | (uintptr_t)c.q_down) & 7u)
        return fail(MOE_ERR_INVALID_ARG, "canonical codes must be 8-byte aligned");
    const Fp8Layout L = fp8_layout(sh);
    const int M = n_mats(sh);
    if (fp8_bytes < L.stride * (size_t)M) return fail(MOE_ERR_WORKSPACE, "FP8 buffer too small");
    const long long rows = (long long)M * (2 * sh.inter + sh.hidden);
    const dim3 grid((unsigned)((rows + 3) / 4));
    if (sh.bits == 8)
        hipLaunchKernelGGL(pack_fp8_kernel<8>, grid, dim3(256), 0, (hipStream_t)stream, c, sh.hidden, sh.inter, M, L,
                           (uint8_t*)fp8);
    else
        hipLaunchKernelGGL(pack_fp8_kernel<4>, grid, dim3(256), 0, (hipStream_t)stream, c, sh.hidden, sh.inter, M, L,
                           (uint8_t*)fp8);
    return check_launch("pack_fp8_kernel");
}

extern "C" size_t moe_prefill_fp8_workspace_bytes(const moe_shape* shape, int32_t T) {
    if (validate_shape(shape) != MOE_OK || T < 1) return 0;
    return fp8_ws_layout(*shape, T).total;
}

extern "C" moe_status moe_experts_prefill_fp8(const moe_shape* shape, const void* experts_fp8, const uint16_t* x,
                                              int32_t T, const int32_t* ids, void* ws, size_t ws_bytes, float* y,
                                              void* stream) {
    clear_error();
    moe_status st = validate_shape(shape);
    if (st != MOE_OK) return st;
    if (T < 1) return fail(MOE_ERR_INVALID_ARG, "T = %d, need T >= 1", T);
    if (!experts_fp8 || !x || !ids || !ws || !y || ((uintptr_t)experts_fp8 & 255u) || !aligned16(x) ||
        !aligned16(ws) || !aligned16(y))
        return fail(MOE_ERR_INVALID_ARG, "NULL or unaligned pointer");
    const moe_shape& sh = *shape;
    const Fp8Ws W = fp8_ws_layout(sh, T);
    if (ws_bytes < W.total)
        return fail(MOE_ERR_WORKSPACE, "FP8 prefill workspace too small (%zu < %zu)", ws_bytes, W.total);
    const Fp8Layout L = fp8_layout(sh);
    const int S = n_slots(sh), H = sh.hidden, I = sh.inter, M = n_mats(sh);
    const size_t P = (size_t)T * S;
    // the GEMMs address activation rows and expert segments with 32-bit byte offsets
    if ((size_t)T * L.Hp > 0xFFFF0000u || P * L.Ip > 0xFFFF0000u || L.stride > 0xFFFF0000u)
        return fail(MOE_ERR_UNSUPPORTED, "T = %d too large for this shape (32-bit row offsets)", T);
    int max_lds = 0, dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
        return fail(MOE_ERR_HIP, "cannot query the device's LDS size");
    if (max_lds < RING8 + 4096)
        return fail(MOE_ERR_UNSUPPORTED, "the FP8 GEMM needs %d bytes of LDS per workgroup, the device has %d",
                    RING8 + 4096, max_lds);
    hipStream_t hs = (hipStream_t)stream;
    char* w = (char*)ws;
    if ((st = launch_prefill_dispatch(sh, T, ids, W.D, w, y, hs)) != MOE_OK) return st;
    uint8_t* x8 = (uint8_t*)(w + W.x8);
    float* xs = (float*)(w + W.xs);
    uint16_t* hbuf = (uint16_t*)(w + W.h);
    uint8_t* h8 = (uint8_t*)(w + W.h8);
    float* hsc = (float*)(w + W.hs);
    hipLaunchKernelGGL(quant_rows_fp8_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, hs, x, (long long)T,
                       (const int32_t*)nullptr, H, L.Hp, x8, xs);
    if ((st = check_launch("quant_rows_fp8_kernel<x>")) != MOE_OK) return st;
    Fp8GemmArgs ga;
    ga.w8 = (const uint8_t*)experts_fp8;
    ga.L = L;
    ga.H = H;
    ga.I = I;
    ga.S = S;
    ga.a8 = x8;
    ga.ascale = xs;
    ga.ntiles = (const int32_t*)(w + W.D.ntiles);
    ga.tiles = (const Tile*)(w + W.D.tiles);
    ga.order = (const int32_t*)(w + W.D.order);
    ga.hbuf = hbuf;
    ga.y = y;
    hipLaunchKernelGGL(fp8_gemm_kernel<true>, dim3(xcd_grid(W.D.max_tiles, (I + 127) / 128)), dim3(256), RING8, hs,
                       ga);
    if ((st = check_launch("fp8_gemm_kernel<gate/up>")) != MOE_OK) return st;
    hipLaunchKernelGGL(quant_rows_fp8_kernel, dim3((unsigned)((P + 3) / 4)), dim3(256), 0, hs, hbuf, (long long)P,
                       (const int32_t*)(w + W.D.offsets) + M, I, L.Ip, h8, hsc);
    if ((st = check_launch("quant_rows_fp8_kernel<h>")) != MOE_OK) return st;
    ga.a8 = h8;
    ga.ascale = hsc;
    hipLaunchKernelGGL(fp8_gemm_kernel<false>, dim3(xcd_grid(W.D.max_tiles, (H + NB8 - 1) / NB8)), dim3(256), RING8, hs,
                       ga);
    return check_launch("fp8_gemm_kernel<down>");
}
