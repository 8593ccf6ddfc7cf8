// attn_mask_compile: host-side MaskInfo preprocessing.
//
// "Lecture 13 - Pallas Kernels and Splash Attention" (CMU 11-868 notes),
// sections 6.1-6.2 and 6.4: the mask is cut into block_q x block_kv blocks;
// blocks without an allowed element are skipped, blocks where every element
// is allowed need no mask, the rest are partial.  The execution table lists
// the active blocks row by row, shares one stored pattern between partial
// blocks with equal patterns (mask_next), and flags the first / last active
// block of each row (bounds_start / bounds_end).  Section 6.6 stores one byte
// per pattern element.
//
// How it is computed here (not by scanning all L_q x L_kv elements):
//   * Without segment ids the allowed keys of query row i form one interval
//     [lo(i), hi(i)] (causal and window bounds), so a block's allowed count
//     is a sum of interval overlaps over its rows.
//   * With segment ids, seg_kv is run-length encoded once; the count for a
//     row adds the overlap of each run with the row's interval whose id
//     equals seg_q[i].
//   * Only the columns between the smallest lo and the largest hi of a block
//     row are visited.
//   * Partial patterns are materialised, hashed (FNV-1a) and deduplicated
//     with a byte comparison, numbered by first appearance in active order.
//   * row_order: rows sorted by active count, longest first, stable.

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <new>
#include <unordered_map>
#include <vector>

#include "errors.h"
#include "splash.h"

namespace {

struct Run {
  int64_t start, end;  // [start, end)
  int32_t id;
};

struct MaskSpec {
  int64_t Lq, Lkv, bq, bkv;
  int64_t qoff;                 // key position of query row 0
  bool causal;
  int64_t wl, wr;
  const int32_t* sq;
  const int32_t* skv;
  std::vector<Run> runs;        // runs of seg_kv
  std::vector<int32_t> run_of;  // key -> index of its run

  // Allowed keys of row i before the segment test: [lo, hi] (empty if lo>hi).
  // Row i sits at key position qoff + i.
  void interval(int64_t i, int64_t* lo, int64_t* hi) const {
    const int64_t pos = qoff + i;
    int64_t a = 0, b = Lkv - 1;
    if (causal) b = std::min(b, pos);
    if (wl >= 0) a = std::max(a, pos - wl);
    if (wr >= 0) b = std::min(b, pos + wr);
    *lo = a;
    *hi = b;
  }

  // Number of allowed keys of row i within [a, b] (a, b valid key indices).
  int64_t count_row(int64_t i, int64_t a, int64_t b) const {
    if (a > b) return 0;
    if (!sq) return b - a + 1;
    const int32_t id = sq[i];
    int64_t n = 0;
    for (size_t r = static_cast<size_t>(run_of[a]); r < runs.size(); ++r) {
      const Run& run = runs[r];
      if (run.start > b) break;
      if (run.id != id) continue;
      n += std::min(run.end - 1, b) - std::max(run.start, a) + 1;
    }
    return n;
  }

  // Writes row i's allowed bytes over keys [k0, k0 + bkv) into dst.
  void pattern_row(int64_t i, int64_t k0, uint8_t* dst) const {
    std::memset(dst, 0, static_cast<size_t>(bkv));
    if (i >= Lq) return;
    int64_t lo, hi;
    interval(i, &lo, &hi);
    const int64_t a = std::max(lo, k0);
    const int64_t b = std::min(hi, k0 + bkv - 1);
    for (int64_t j = a; j <= b; ++j)
      dst[j - k0] = (!sq || sq[i] == skv[j]) ? 1 : 0;
  }
};

struct Compiled {
  int64_t nq = 0, nkv = 0;
  std::vector<int8_t> block_mask;
  std::vector<int32_t> rows, cols, mask_next, row_ptr, row_order;
  std::vector<int8_t> code;
  std::vector<uint8_t> bounds;
  std::vector<uint8_t> patterns;  // n_patterns * bq * bkv
  int64_t n_patterns = 0;
  int64_t n_partial = 0;
};

uint64_t fnv1a(const uint8_t* p, size_t n) {
  uint64_t h = 1469598103934665603ull;
  for (size_t i = 0; i < n; ++i) {
    h ^= p[i];
    h *= 1099511628211ull;
  }
  return h;
}

int compile(const splash_mask_desc& d, Compiled* out) {
  MaskSpec m;
  m.Lq = d.L_q;
  m.Lkv = d.L_kv;
  m.qoff = d.q_offset;
  m.bq = d.block_q;
  m.bkv = d.block_kv;
  m.causal = d.causal != 0;
  m.wl = d.window_left;
  m.wr = d.window_right;
  m.sq = d.seg_q;
  m.skv = d.seg_kv ? d.seg_kv : d.seg_q;
  if (!m.sq) m.skv = nullptr;

  const int64_t nq = (m.Lq + m.bq - 1) / m.bq;
  const int64_t nkv = (m.Lkv + m.bkv - 1) / m.bkv;
  if (nq * nkv > INT32_MAX || m.bq * m.bkv > INT32_MAX)
    return splash::fail(SPLASH_ESHAPE, "attn_mask_compile: %lld x %lld blocks is too many",
                        static_cast<long long>(nq), static_cast<long long>(nkv));
  out->nq = nq;
  out->nkv = nkv;

  if (m.sq && m.Lkv > 0) {
    m.run_of.resize(static_cast<size_t>(m.Lkv));
    int64_t s = 0;
    while (s < m.Lkv) {
      int64_t e = s + 1;
      while (e < m.Lkv && m.skv[e] == m.skv[s]) ++e;
      const int32_t idx = static_cast<int32_t>(m.runs.size());
      m.runs.push_back({s, e, m.skv[s]});
      for (int64_t j = s; j < e; ++j) m.run_of[j] = idx;
      s = e;
    }
  }

  out->block_mask.assign(static_cast<size_t>(nq * nkv), 0);
  out->row_ptr.assign(static_cast<size_t>(nq + 1), 0);
  const int64_t full = m.bq * m.bkv;
  const size_t pat_bytes = static_cast<size_t>(full);
  std::vector<uint8_t> pat(pat_bytes);
  std::unordered_map<uint64_t, std::vector<int32_t>> seen;

  for (int64_t r = 0; r < nq; ++r) {
    const int64_t i0 = r * m.bq;
    const int64_t i1 = std::min(i0 + m.bq, m.Lq);  // valid rows [i0, i1)
    int64_t cmin = nkv, cmax = -1;
    for (int64_t i = i0; i < i1; ++i) {
      int64_t lo, hi;
      m.interval(i, &lo, &hi);
      if (lo > hi) continue;
      cmin = std::min(cmin, lo / m.bkv);
      cmax = std::max(cmax, hi / m.bkv);
    }
    const size_t first = out->rows.size();
    for (int64_t c = cmin; c <= cmax; ++c) {
      const int64_t k0 = c * m.bkv;
      const int64_t k1 = std::min(k0 + m.bkv, m.Lkv) - 1;  // last valid key
      int64_t count = 0;
      for (int64_t i = i0; i < i1; ++i) {
        int64_t lo, hi;
        m.interval(i, &lo, &hi);
        count += m.count_row(i, std::max(lo, k0), std::min(hi, k1));
      }
      if (count == 0) continue;
      const int8_t code = (count == full) ? 2 : 1;
      out->block_mask[static_cast<size_t>(r * nkv + c)] = code;
      out->rows.push_back(static_cast<int32_t>(r));
      out->cols.push_back(static_cast<int32_t>(c));
      out->code.push_back(code);
      if (code == 2) {
        out->mask_next.push_back(-1);
        continue;
      }
      ++out->n_partial;
      for (int64_t a = 0; a < m.bq; ++a)
        m.pattern_row(i0 + a, k0, pat.data() + a * m.bkv);
      const uint64_t h = fnv1a(pat.data(), pat_bytes);
      std::vector<int32_t>& bucket = seen[h];
      int32_t found = -1;
      for (int32_t idx : bucket) {
        if (std::memcmp(out->patterns.data() + static_cast<size_t>(idx) * pat_bytes,
                        pat.data(), pat_bytes) == 0) {
          found = idx;
          break;
        }
      }
      if (found < 0) {
        found = static_cast<int32_t>(out->n_patterns++);
        bucket.push_back(found);
        out->patterns.insert(out->patterns.end(), pat.begin(), pat.end());
      }
      out->mask_next.push_back(found);
    }
    const size_t n = out->rows.size() - first;
    for (size_t t = 0; t < n; ++t)
      out->bounds.push_back(static_cast<uint8_t>((t == 0 ? 1 : 0) | (t + 1 == n ? 2 : 0)));
    out->row_ptr[static_cast<size_t>(r + 1)] = static_cast<int32_t>(out->rows.size());
  }
  if (out->rows.size() > static_cast<size_t>(INT32_MAX))
    return splash::fail(SPLASH_ESHAPE, "attn_mask_compile: too many active blocks");

  out->row_order.resize(static_cast<size_t>(nq));
  for (int64_t r = 0; r < nq; ++r) out->row_order[static_cast<size_t>(r)] = static_cast<int32_t>(r);
  const std::vector<int32_t>& rp = out->row_ptr;
  std::stable_sort(out->row_order.begin(), out->row_order.end(), [&rp](int32_t a, int32_t b) {
    return (rp[a + 1] - rp[a]) > (rp[b + 1] - rp[b]);
  });
  return SPLASH_OK;
}

template <typename T>
void copy_out(T* dst, const std::vector<T>& src) {
  if (dst && !src.empty()) std::memcpy(dst, src.data(), src.size() * sizeof(T));
}

}  // namespace

extern "C" int attn_mask_compile(const splash_mask_desc* desc, splash_mask_sizes* sizes,
                                 splash_mask_tables* tables) {
  splash::clear_error();
  if (!desc || !sizes) return splash::fail(SPLASH_EINVAL, "attn_mask_compile: NULL desc or sizes");
  const splash_mask_desc& d = *desc;
  if (d.L_q < 0 || d.L_kv < 0)
    return splash::fail(SPLASH_EINVAL, "attn_mask_compile: negative length (L_q=%d, L_kv=%d)",
                        d.L_q, d.L_kv);
  if (d.block_q <= 0 || d.block_kv <= 0)
    return splash::fail(SPLASH_EINVAL, "attn_mask_compile: block sizes must be > 0 (%d, %d)",
                        d.block_q, d.block_kv);
  if (d.causal != 0 && d.causal != 1)
    return splash::fail(SPLASH_EINVAL, "attn_mask_compile: causal must be 0 or 1");
  if (d.q_offset < 0)
    return splash::fail(SPLASH_EINVAL, "attn_mask_compile: q_offset must be >= 0 (%d)", d.q_offset);
  if (d.window_left < -1 || d.window_right < -1)
    return splash::fail(SPLASH_EINVAL, "attn_mask_compile: window must be -1 or >= 0 (%d, %d)",
                        d.window_left, d.window_right);
  if (d.seg_q && !d.seg_kv && d.L_q != d.L_kv)
    return splash::fail(SPLASH_EINVAL,
                        "attn_mask_compile: seg_kv is NULL but L_kv (%d) != L_q (%d)", d.L_kv,
                        d.L_q);
  if (!d.seg_q && d.seg_kv)
    return splash::fail(SPLASH_EINVAL, "attn_mask_compile: seg_kv given without seg_q");
  try {
    Compiled c;
    const int rc = compile(d, &c);
    if (rc != SPLASH_OK) return rc;
    splash_mask_sizes s;
    s.n_q_blocks = static_cast<int32_t>(c.nq);
    s.n_kv_blocks = static_cast<int32_t>(c.nkv);
    s.n_active = static_cast<int32_t>(c.rows.size());
    s.n_partial = static_cast<int32_t>(c.n_partial);
    s.n_patterns = static_cast<int32_t>(c.n_patterns);
    if (!tables) {
      *sizes = s;
      return SPLASH_OK;
    }
    if (std::memcmp(&s, sizes, sizeof(s)) != 0)
      return splash::fail(SPLASH_ESHAPE,
                          "attn_mask_compile: sizes (%d,%d,%d,%d,%d) do not match this mask "
                          "(%d,%d,%d,%d,%d)",
                          sizes->n_q_blocks, sizes->n_kv_blocks, sizes->n_active,
                          sizes->n_partial, sizes->n_patterns, s.n_q_blocks, s.n_kv_blocks,
                          s.n_active, s.n_partial, s.n_patterns);
    copy_out(tables->block_mask, c.block_mask);
    copy_out(tables->active_rows, c.rows);
    copy_out(tables->active_cols, c.cols);
    copy_out(tables->block_code, c.code);
    copy_out(tables->mask_next, c.mask_next);
    copy_out(tables->bounds, c.bounds);
    copy_out(tables->row_ptr, c.row_ptr);
    copy_out(tables->row_order, c.row_order);
    copy_out(tables->partial_mask_blocks, c.patterns);
    return SPLASH_OK;
  } catch (const std::bad_alloc&) {
    return splash::fail(SPLASH_ENOMEM, "attn_mask_compile: out of host memory");
  } catch (...) {
    return splash::fail(SPLASH_EINTERNAL, "attn_mask_compile: unexpected exception");
  }
}

// Column-major view of an execution table: a counting sort of the row-major
// active list by kv-block column (rows stay ascending inside a column).
extern "C" int attn_mask_columns(int32_t n_q_blocks, int32_t n_kv_blocks, int32_t n_active,
                                 const int32_t* row_ptr, const int32_t* active_cols,
                                 int32_t* col_ptr, int32_t* col_rows, int32_t* col_entry) {
  splash::clear_error();
  if (n_q_blocks < 0 || n_kv_blocks < 0 || n_active < 0)
    return splash::fail(SPLASH_EINVAL, "attn_mask_columns: negative size");
  if (!row_ptr || !col_ptr || (n_active > 0 && (!active_cols || !col_rows || !col_entry)))
    return splash::fail(SPLASH_EINVAL, "attn_mask_columns: NULL array");
  if (row_ptr[0] != 0 || row_ptr[n_q_blocks] != n_active)
    return splash::fail(SPLASH_EINVAL, "attn_mask_columns: row_ptr must run from 0 to n_active");
  for (int32_t r = 0; r < n_q_blocks; ++r) {
    if (row_ptr[r + 1] < row_ptr[r])
      return splash::fail(SPLASH_EINVAL, "attn_mask_columns: row_ptr decreases at row %d", r);
    for (int32_t e = row_ptr[r]; e < row_ptr[r + 1]; ++e) {
      const int32_t c = active_cols[e];
      if (c < 0 || c >= n_kv_blocks || (e > row_ptr[r] && c <= active_cols[e - 1]))
        return splash::fail(SPLASH_EINVAL,
                            "attn_mask_columns: columns of row %d must ascend within [0, %d)", r,
                            n_kv_blocks);
    }
  }
  for (int32_t c = 0; c <= n_kv_blocks; ++c) col_ptr[c] = 0;
  for (int32_t e = 0; e < n_active; ++e) ++col_ptr[active_cols[e] + 1];
  for (int32_t c = 0; c < n_kv_blocks; ++c) col_ptr[c + 1] += col_ptr[c];
  std::vector<int32_t> fill(col_ptr, col_ptr + n_kv_blocks);
  for (int32_t r = 0; r < n_q_blocks; ++r) {
    for (int32_t e = row_ptr[r]; e < row_ptr[r + 1]; ++e) {
      const int32_t x = fill[active_cols[e]]++;
      col_rows[x] = r;
      col_entry[x] = e;
    }
  }
  return SPLASH_OK;
}

extern "C" int attn_mask_column_order(int32_t n_kv_blocks, const int32_t* col_ptr, int32_t* col_order) {
  splash::clear_error();
  if (n_kv_blocks < 0) return splash::fail(SPLASH_EINVAL, "attn_mask_column_order: negative size");
  if (!col_ptr || (n_kv_blocks > 0 && !col_order))
    return splash::fail(SPLASH_EINVAL, "attn_mask_column_order: NULL array");
  if (col_ptr[0] != 0) return splash::fail(SPLASH_EINVAL, "attn_mask_column_order: col_ptr must start at 0");
  for (int32_t c = 0; c < n_kv_blocks; ++c)
    if (col_ptr[c + 1] < col_ptr[c])
      return splash::fail(SPLASH_EINVAL, "attn_mask_column_order: col_ptr decreases at column %d", c);
  for (int32_t c = 0; c < n_kv_blocks; ++c) col_order[c] = c;
  std::stable_sort(col_order, col_order + n_kv_blocks, [col_ptr](int32_t a, int32_t b) {
    return col_ptr[a + 1] - col_ptr[a] > col_ptr[b + 1] - col_ptr[b];
  });
  return SPLASH_OK;
}
