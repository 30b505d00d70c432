// Host-side canonicaliser of block-sparse metadata (attn_blockmask_build).
//
// A raw pattern lists, per query block, the key blocks it attends to
// ("Exact Blocks, Rings, and Sparsity", section 5: the active set C_a of query
// tile a).  Raw lists may be unordered, hold repeats, be empty or, under
// causal, name future blocks ("block-sparse attention patterns": test
// ordering, duplicates, empty rows and partial blocks; a duplicate must not
// count a key twice).  The canonical form the kernels consume keeps each row
// sorted and unique and drops future blocks when causal, so a kernel visits a
// tile at most once and never visits a tile with no allowed pair.
//
// Pair counts are computed from tile geometry: a tile of query block qb and
// key block kb holds rows(qb) x cols(kb) valid pairs (the last block holds
// N - (nqb-1)*b tokens), and the causal diagonal tile holds n(n+1)/2.
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <vector>

#include "bsattn.h"

namespace {

int64_t valid_in_block(int64_t blk, int64_t N, int64_t block) {
    const int64_t lo = blk * block;
    const int64_t hi = std::min(N, lo + block);
    return hi > lo ? hi - lo : 0;
}

}  // namespace

extern "C" int attn_blockmask_build(const int32_t* raw_row_ptr, const int32_t* raw_col,
                                    int64_t meta_heads, int64_t N, int64_t block, int causal,
                                    int32_t* row_ptr, int32_t* col, uint8_t* flags,
                                    int64_t capacity, int64_t* nnz, int64_t* allowed_pairs,
                                    int64_t* executed_tile_pairs) {
    if (!raw_row_ptr || !row_ptr || !nnz || !allowed_pairs || !executed_tile_pairs)
        return ATTN_EINVAL;
    if (meta_heads < 1 || N < 1 || block < 1 || N > INT32_MAX || meta_heads > INT32_MAX)
        return ATTN_EINVAL;
    if (causal != 0 && causal != 1) return ATTN_EINVAL;
    if (capacity < 0 || (capacity > 0 && (!col || !flags))) return ATTN_EINVAL;
    const int64_t nqb = (N + block - 1) / block;
    const int64_t nrows = meta_heads * nqb;
    if (nrows > INT32_MAX) return ATTN_EINVAL;
    if (raw_row_ptr[0] != 0) return ATTN_EINVAL;
    for (int64_t r = 0; r < nrows; ++r)
        if (raw_row_ptr[r + 1] < raw_row_ptr[r]) return ATTN_EINVAL;
    const int64_t raw_nnz = raw_row_ptr[nrows];
    if (raw_nnz > 0 && !raw_col) return ATTN_EINVAL;
    for (int64_t e = 0; e < raw_nnz; ++e)
        if (raw_col[e] < 0 || raw_col[e] >= nqb) return ATTN_EINVAL;

    const bool partial = (N % block) != 0;
    // One bit per key block marks membership; the row's entries are then read
    // back in increasing order, which sorts and deduplicates in O(raw + listed).
    std::vector<uint8_t> seen(static_cast<size_t>(nqb), 0);
    std::vector<int32_t> row;
    row.reserve(static_cast<size_t>(nqb));
    int64_t out = 0;
    bool overflow = false;
    row_ptr[0] = 0;
    for (int64_t h = 0; h < meta_heads; ++h) {
        int64_t allowed = 0, tiles = 0;
        for (int64_t qb = 0; qb < nqb; ++qb) {
            const int64_t r = h * nqb + qb;
            row.clear();
            for (int64_t e = raw_row_ptr[r]; e < raw_row_ptr[r + 1]; ++e) {
                const int32_t kb = raw_col[e];
                if (causal && kb > qb) continue;
                if (!seen[kb]) {
                    seen[kb] = 1;
                    row.push_back(kb);
                }
            }
            std::sort(row.begin(), row.end());
            const int64_t nrow_q = valid_in_block(qb, N, block);
            for (int32_t kb : row) {
                seen[kb] = 0;
                uint8_t f = 0;
                if (causal && kb == qb && block > 1) f |= ATTN_FLAG_DIAGONAL;
                if (partial && kb == nqb - 1) f |= ATTN_FLAG_PARTIAL;
                if (causal && kb == qb) {
                    allowed += nrow_q * (nrow_q + 1) / 2;
                } else {
                    allowed += nrow_q * valid_in_block(kb, N, block);
                }
                if (out < capacity) {
                    col[out] = kb;
                    flags[out] = f;
                } else {
                    overflow = true;
                }
                ++out;
            }
            tiles += static_cast<int64_t>(row.size());
            if (out > INT32_MAX) return ATTN_EINVAL;
            row_ptr[r + 1] = static_cast<int32_t>(out);
        }
        allowed_pairs[h] = allowed;
        executed_tile_pairs[h] = tiles;
    }
    *nnz = out;
    return overflow ? ATTN_ECAPACITY : ATTN_OK;
}

// Transpose of canonical (or any valid) CSR metadata: for each key block, the
// query blocks whose lists name it, in increasing order.  The backward's dK/dV
// pass owns a key block and visits exactly these query blocks ("Exact Blocks,
// Rings, and Sparsity", section 3: the dK/dV reduction runs over queries).
extern "C" int attn_blockmask_transpose(const int32_t* row_ptr, const int32_t* col, int64_t meta_heads,
                                        int64_t N, int64_t block, int32_t* t_row_ptr, int32_t* t_col,
                                        int64_t capacity) {
    if (!row_ptr || !t_row_ptr) return ATTN_EINVAL;
    if (meta_heads < 1 || N < 1 || block < 1 || N > INT32_MAX || meta_heads > INT32_MAX) return ATTN_EINVAL;
    if (capacity < 0) return ATTN_EINVAL;
    const int64_t nb = (N + block - 1) / block;
    const int64_t nrows = meta_heads * nb;
    if (nrows > INT32_MAX) return ATTN_EINVAL;
    if (row_ptr[0] != 0) return ATTN_EINVAL;
    for (int64_t r = 0; r < nrows; ++r)
        if (row_ptr[r + 1] < row_ptr[r]) return ATTN_EINVAL;
    const int64_t nnz = row_ptr[nrows];
    if (nnz > 0 && !col) return ATTN_EINVAL;
    for (int64_t e = 0; e < nnz; ++e)
        if (col[e] < 0 || col[e] >= nb) return ATTN_EINVAL;
    // counts per (meta head, key block), then offsets
    std::vector<int64_t> fill(static_cast<size_t>(nrows + 1), 0);
    for (int64_t h = 0; h < meta_heads; ++h)
        for (int64_t qb = 0; qb < nb; ++qb)
            for (int64_t e = row_ptr[h * nb + qb]; e < row_ptr[h * nb + qb + 1]; ++e) ++fill[h * nb + col[e] + 1];
    for (int64_t r = 0; r < nrows; ++r) fill[r + 1] += fill[r];
    for (int64_t r = 0; r <= nrows; ++r) t_row_ptr[r] = static_cast<int32_t>(fill[r]);
    if (nnz > capacity) return ATTN_ECAPACITY;
    if (nnz > 0 && !t_col) return ATTN_EINVAL;
    // query blocks in increasing order keep every transposed row sorted
    for (int64_t h = 0; h < meta_heads; ++h)
        for (int64_t qb = 0; qb < nb; ++qb)
            for (int64_t e = row_ptr[h * nb + qb]; e < row_ptr[h * nb + qb + 1]; ++e)
                t_col[fill[h * nb + col[e]]++] = static_cast<int32_t>(qb);
    return ATTN_OK;
}
