// concat_mla_k: MLA key rows assembled from their "nope" and "rope" parts.
//
// Page on FlashInfer's concat_mla_k with FP8 inputs, sections 1-3: a key row
// is 128 nope elements followed by 64 rope elements, for 1-byte (E4M3, E5M2)
// or 2-byte (BF16, FP16) elements; the bytes are moved unchanged.
//   k_nope [T, H, 128], k_rope [T, R, 64] with R == 1 (shared by the token's
//   heads) or R == H, k [T, H, 192]:  k[t,h] = k_nope[t,h] ++ k_rope[t, R == 1 ? 0 : h]
//
// HBM-bound byte move.  Every row boundary is a multiple of 16 bytes for both
// element sizes (128, 64 and 192 elements), so each lane moves 16-byte
// chunks: an output row is 12 (1-byte) or 24 (2-byte) chunks, the first 8 (16)
// from the nope row, the rest from the rope row.  Consecutive lanes write
// consecutive chunks of k (fully coalesced stores, non-temporal: k is not read
// back here); nope chunks are read once (non-temporal), rope rows are read by
// every head of their token and stay in cache.

#include "device_common.h"
#include "launch.h"

namespace fp8g {

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

constexpr int CONCAT_THREADS = 256;

template <int E>   // element size in bytes
__global__ __launch_bounds__(CONCAT_THREADS) void concat_mla_k_kernel(v4u* __restrict__ k, const v4u* __restrict__ nope,
                                                                      const v4u* __restrict__ rope, int64_t rows,
                                                                      int64_t heads, int64_t rope_heads) {
    constexpr int CPR = 12 * E, CN = 8 * E, CR = 4 * E;   // 16-byte chunks: per row, nope, rope
    const int64_t total = rows * CPR;
    const int64_t step = (int64_t)gridDim.x * CONCAT_THREADS;
    for (int64_t c = (int64_t)blockIdx.x * CONCAT_THREADS + threadIdx.x; c < total; c += step) {
        const int64_t row = c / CPR;                       // row = t * H + h
        const int j = (int)(c - row * CPR);
        v4u v;
        if (j < CN) {
            v = __builtin_nontemporal_load(nope + row * CN + j);
        } else {
            const int64_t t = row / heads;
            const int64_t rrow = rope_heads == 1 ? t : row;   // R == H: same row index as k
            v = rope[rrow * CR + (j - CN)];
        }
        __builtin_nontemporal_store(v, k + c);
    }
}

hipError_t launch_concat_mla_k(void* k, const void* k_nope, const void* k_rope, int64_t tokens, int64_t heads,
                               int64_t rope_heads, int elem_bytes, hipStream_t stream) {
    const int64_t rows = tokens * heads;
    if (rows == 0) return hipSuccess;
    const int64_t total = rows * 12 * elem_bytes;
    int64_t blocks = (total + CONCAT_THREADS - 1) / CONCAT_THREADS;
    if (blocks > 8192) blocks = 8192;   // grid-stride beyond: 32 workgroups per CU
    const dim3 grid((unsigned)blocks), block(CONCAT_THREADS);
    if (elem_bytes == 1)
        concat_mla_k_kernel<1><<<grid, block, 0, stream>>>(static_cast<v4u*>(k), static_cast<const v4u*>(k_nope),
                                                           static_cast<const v4u*>(k_rope), rows, heads, rope_heads);
    else
        concat_mla_k_kernel<2><<<grid, block, 0, stream>>>(static_cast<v4u*>(k), static_cast<const v4u*>(k_nope),
                                                           static_cast<const v4u*>(k_rope), rows, heads, rope_heads);
    return hipGetLastError();
}

}  // namespace fp8g
