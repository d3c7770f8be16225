/* Packed CPU oracle of the forward pass of Monodratic routed sparse causal attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Loaded (ctypes, through oracle/packed.py) by tests/ and by the
 * cpu_baseline leg of bench.py; never by the HIP library or its Python binding, and it shares no
 * code with them.  It computes what the NumPy oracle (mdr_oracle.py) computes -- the same steps, in
 * the same order, with the same readings of the pages -- as plain single-threaded loops, gathering
 * only the selected tokens instead of building a dense mask, so that its running time is a
 * meaningful CPU figure.  The pages' own timing is of such a packed CPU implementation of the
 * routing (aitechinspire.com write-up of Monodratic, "Scaling behavior and implementation notes";
 * remio.ai, "Monodratic claims learned routing can make sparse causal attention more selective",
 * section "Why learned product-hash routing matters now").
 *
 * One call handles one (batch, head) and the query tokens [t0, t1):
 *   1. block key summaries: the mean of each block's post-RoPE key rows (fp32);
 *   2. per block, a product address: per subspace the argmax of the code logits
 *      <codebook[g, c], summary> + bias[g, c] (first maximum wins), combined as a mixed-radix
 *      number with subspace 0 most significant (remio.ai, section "Monodratic turns sparse
 *      attention into a retrieval decision");
 *   3. posting lists: blocks i < nb - L filed under their address in ascending order; query block
 *      j sees, per address, the newest `capacity` blocks i <= j - L, newest first (same section:
 *      bounded causal posting lists; a block never serves a query placed before it);
 *   4. per token: the query's code logits, the score of every address (sum over subspaces, in
 *      order, of the logit of its digit), the top-P addresses (ties to the smaller address), their
 *      views concatenated in probe rank order and cut at M, a rerank by <q, summary> and the top-R
 *      candidates (ties to the smaller block) (aitechinspire.com, "What's the core idea?"; remio.ai,
 *      "Why learned product-hash routing matters now": the index is the coarse filter, the probes
 *      generate candidates, the rerank makes the finer choice);
 *   5. exact softmax over the tokens of the selected blocks and the causal local window (the L most
 *      recent blocks, the current one up to the token), scale 1/sqrt(D), in fp64 (aitechinspire.com,
 *      "Snapshot: key facts from the report": exact attention after selection).
 * Routing decisions are taken in fp32, as in the NumPy oracle; only the order of the fp32 additions
 * differs from it (near-ties may then be decided differently, and are compared as such).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Step 1: mean of each block's key rows. */
static void block_summaries(const float* k, int nb, int D, int block, float* ksum) {
  for (int i = 0; i < nb; ++i)
    for (int d = 0; d < D; ++d) {
      float acc = 0.f;
      for (int r = 0; r < block; ++r) acc += k[((size_t)i * block + r) * D + d];
      ksum[(size_t)i * D + d] = acc / (float)block;
    }
}

/* Steps 2 and 4: code logits of one vector x, mu[g * C + c] = <codebook[g, c], x> + bias[g, c]. */
static void code_logits(const float* x, const float* cb, const float* bias, int G, int C, int D, float* mu) {
  for (int gc = 0; gc < G * C; ++gc) {
    float acc = 0.f;
    for (int d = 0; d < D; ++d) acc += cb[(size_t)gc * D + d] * x[d];
    mu[gc] = bias ? acc + bias[gc] : acc;
  }
}

/* Step 2: product address from the code logits, per subspace the first maximum. */
static int product_address(const float* mu, int G, int C) {
  int a = 0;
  for (int g = 0; g < G; ++g) {
    int best = 0;
    for (int c = 1; c < C; ++c)
      if (mu[g * C + c] > mu[g * C + best]) best = c;
    a = a * C + best;
  }
  return a;
}

/* Entry (score, index) ranks before (score2, index2): larger score first, smaller index on ties. */
static int ranks_before(float s, int i, float s2, int i2) { return s > s2 || (s == s2 && i < i2); }

/* Insert (s, i) into the sorted top list (val, idx) of capacity cap holding *n entries. */
static void top_insert(float* val, int* idx, int* n, int cap, float s, int i) {
  int p = *n < cap ? *n : cap;
  if (p == cap && !ranks_before(s, i, val[cap - 1], idx[cap - 1])) return;
  if (p == cap) p = cap - 1;
  while (p > 0 && ranks_before(s, i, val[p - 1], idx[p - 1])) {
    val[p] = val[p - 1];
    idx[p] = idx[p - 1];
    --p;
  }
  val[p] = s;
  idx[p] = i;
  if (*n < cap) ++*n;
}

/* Forward of one (batch, head) for query tokens [t0, t1).  q, k, v: [S, D] fp32 rows (bf16 inputs
 * upcast); codebook [G, C, D]; bias [G, C] or NULL; max_cand 0 means probes * capacity.
 * sel: [(t1 - t0), remote] selected blocks in rank order, -1 beyond the last; out: [(t1 - t0), D].
 * Returns 0, or -1 on invalid sizes, -2 when out of memory. */
int mdr_packed_forward(const float* q, const float* k, const float* v, int S, int D, const float* codebook,
                       const float* bias, int G, int C, int block, int capacity, int probes, int max_cand,
                       int remote, int local, int t0, int t1, int32_t* sel, double* out) {
  if (S < 1 || D < 1 || block < 1 || S % block || G < 1 || C < 1 || capacity < 1 || probes < 1 || remote < 0 ||
      local < 1 || t0 < 0 || t1 > S || t0 > t1)
    return -1;
  int A = 1;
  for (int g = 0; g < G; ++g) {
    if (A > (1 << 24) / C) return -1;
    A *= C;
  }
  const int nb = S / block, M = max_cand > 0 ? max_cand : probes * capacity;
  const int P = probes < A ? probes : A;
  float* ksum = malloc(sizeof(float) * (size_t)nb * D);
  int* addr = malloc(sizeof(int) * (size_t)nb);
  int* off = calloc((size_t)A + 1, sizeof(int));
  int* idx = malloc(sizeof(int) * (size_t)nb);
  float* mu = malloc(sizeof(float) * (size_t)G * C);
  float* sigma = malloc(sizeof(float) * (size_t)A);
  float* pval = malloc(sizeof(float) * (size_t)P);
  int* pidx = malloc(sizeof(int) * (size_t)P);
  int* cand = malloc(sizeof(int) * (size_t)(M > 0 ? M : 1));
  float* rval = malloc(sizeof(float) * (size_t)(remote > 0 ? remote : 1));
  int* ridx = malloc(sizeof(int) * (size_t)(remote > 0 ? remote : 1));
  const int maxkeys = (remote + local) * block;
  int* keys = malloc(sizeof(int) * (size_t)maxkeys);
  double* sc = malloc(sizeof(double) * (size_t)maxkeys);
  int rc = 0;
  if (!ksum || !addr || !off || !idx || !mu || !sigma || !pval || !pidx || !cand || !rval || !ridx || !keys || !sc) {
    rc = -2;
    goto done;
  }
  /* steps 1-2 */
  block_summaries(k, nb, D, block, ksum);
  for (int i = 0; i < nb; ++i) {
    code_logits(ksum + (size_t)i * D, codebook, bias, G, C, D, mu);
    addr[i] = product_address(mu, G, C);
  }
  /* step 3: CSR of the lists, blocks i < nb - L in ascending order */
  const int nfiled = nb > local ? nb - local : 0;
  for (int i = 0; i < nfiled; ++i) off[addr[i] + 1]++;
  for (int a = 0; a < A; ++a) off[a + 1] += off[a];
  {
    int* cur = malloc(sizeof(int) * (size_t)A);
    if (!cur) {
      rc = -2;
      goto done;
    }
    memcpy(cur, off, sizeof(int) * (size_t)A);
    for (int i = 0; i < nfiled; ++i) idx[cur[addr[i]]++] = i;
    free(cur);
  }
  const double scale = 1.0 / sqrt((double)D);
  for (int t = t0; t < t1; ++t) {
    const int j = t / block, cutoff = j - local;
    const float* qt = q + (size_t)t * D;
    /* step 4: probes */
    code_logits(qt, codebook, bias, G, C, D, mu);
    for (int a = 0; a < A; ++a) {
      float s = 0.f;
      int rest = a, div = A;
      for (int g = 0; g < G; ++g) {
        div /= C;
        const int digit = rest / div;
        rest -= digit * div;
        s = g == 0 ? mu[digit] : s + mu[g * C + digit];
      }
      sigma[a] = s;
    }
    int np = 0;
    for (int a = 0; a < A; ++a) top_insert(pval, pidx, &np, P, sigma[a], a);
    /* candidates: each probe's view (newest `capacity` eligible blocks, newest first), cut at M */
    int nc = 0;
    if (cutoff >= 0)
      for (int p = 0; p < np && nc < M; ++p) {
        const int a = pidx[p];
        int taken = 0;
        for (int x = off[a + 1] - 1; x >= off[a] && taken < capacity && nc < M; --x)
          if (idx[x] <= cutoff) {
            cand[nc++] = idx[x];
            ++taken;
          }
      }
    /* rerank: top-R by <q, summary> */
    int nr = 0;
    for (int c = 0; c < nc && remote > 0; ++c) {
      float s = 0.f;
      const float* ks = ksum + (size_t)cand[c] * D;
      for (int d = 0; d < D; ++d) s += ks[d] * qt[d];
      top_insert(rval, ridx, &nr, remote, s, cand[c]);
    }
    int32_t* srow = sel + (size_t)(t - t0) * remote;
    for (int r = 0; r < remote; ++r) srow[r] = r < nr ? ridx[r] : -1;
    /* step 5: the selected blocks' tokens, then the local window up to t */
    int nk = 0;
    for (int r = 0; r < nr; ++r)
      for (int x = 0; x < block; ++x) keys[nk++] = ridx[r] * block + x;
    const int lo = (j - local + 1) * block > 0 ? (j - local + 1) * block : 0;
    for (int x = lo; x <= t; ++x) keys[nk++] = x;
    double mx = -INFINITY;
    for (int n = 0; n < nk; ++n) {
      double s = 0.0;
      const float* kr = k + (size_t)keys[n] * D;
      for (int d = 0; d < D; ++d) s += (double)kr[d] * (double)qt[d];
      sc[n] = s * scale;
      if (sc[n] > mx) mx = sc[n];
    }
    double den = 0.0;
    double* o = out + (size_t)(t - t0) * D;
    for (int d = 0; d < D; ++d) o[d] = 0.0;
    for (int n = 0; n < nk; ++n) {
      const double p = exp(sc[n] - mx);
      den += p;
      const float* vr = v + (size_t)keys[n] * D;
      for (int d = 0; d < D; ++d) o[d] += p * (double)vr[d];
    }
    for (int d = 0; d < D; ++d) o[d] /= den;
  }
done:
  free(ksum);
  free(addr);
  free(off);
  free(idx);
  free(mu);
  free(sigma);
  free(pval);
  free(pidx);
  free(cand);
  free(rval);
  free(ridx);
  free(keys);
  free(sc);
  return rc;
}
