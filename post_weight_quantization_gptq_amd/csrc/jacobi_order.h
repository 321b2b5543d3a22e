// Pair order of the one-sided Jacobi sweeps of the Rayleigh-Ritz step
// (k_ritz in lora.hip), as plain integer code: the kernel builds its LDS
// table from it, and a host-only checker compiles the same header.
#pragma once

#ifdef __HIPCC__
#define JACOBI_HD __host__ __device__
#else
#define JACOBI_HD
#endif

// Pair schedule of one Jacobi sweep over mp (even) columns, built so that a
// unit (the lanes working on one pair) keeps one of its two columns from one
// round to the next nearly always.  Cross level on groups of g columns (first
// g = mp): the group's q = g/2 units each keep a column of the first half and
// take the columns of the second half in cyclic order, q rounds for all q^2
// cross pairs; then each half becomes a group of the next level.  Once q is
// odd the pairs inside each half of q columns follow the circle method on
// q + 1 places (one of them a dummy), q more rounds.  Every pair of columns
// is met once per sweep, and no column is in two pairs of one round.
// Rounds per sweep: the sum of the q's, which is mp less the last q, plus
// that q again when it is odd and above 1; so at most mp.
JACOBI_HD inline int ritz_rounds(int mp) {
  int g = mp, R = 0;
  while (true) {
    const int q = g >> 1;
    R += q;
    if (q & 1) return q > 1 ? R + q : R;
    g = q;
  }
}

// Columns (a, b) of unit u in round ri of a sweep; a < 0: idle this round.
JACOBI_HD inline void ritz_assign(int mp, int ri, int u, int& a, int& b) {
  a = b = -1;
  int g = mp;
  while (true) {
    const int q = g >> 1;
    if (ri < q) {
      const int G = u / q, v = u - G * q;
      if (G < mp / g) {
        a = G * g + v;
        b = G * g + q + (v + ri) % q;
      }
      return;
    }
    ri -= q;
    if (q & 1) {
      if (q == 1 || ri >= q) return;
      const int G = u / q, v = u - G * q, npr = (q - 1) / 2;
      if (G >= mp / g || v >= 2 * npr) return;
      const int half = v / npr, w = v - half * npr;
      // place 0 holds column 0, place i >= 1 column 1 + (i - 1 + ri) mod q,
      // where column q is the dummy; pair j joins places j and q - j
      const int idum = ri == 0 ? q : q - ri, jd = idum < q - idum ? idum : q - idum;
      const int j = w < jd ? w : w + 1, base = G * g + half * q;
      a = base + (j == 0 ? 0 : 1 + (j - 1 + ri) % q);
      b = base + 1 + (q - j - 1 + ri) % q;
      return;
    }
    g = q;
  }
}
