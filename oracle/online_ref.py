"""Pure-Python fp64 twin of the online softmax normaliser, for tiny rows only.

TEST INFRASTRUCTURE ONLY (see the package docstring).  This file states the
online method in the pages' own terms so the tests can check it against the
three-pass oracle in ``oracle.c``: two different algorithms that must reach
the same (m, d) and the same probabilities.

* The element-by-element recurrence, for a running pair (m, d) and a new
  element x:  m' = max(m, x),  d' = d * exp(m - m') + exp(x - m').
  "RMSNorm、Softmax 与在线归约" (notes.kuangjux.top), section "Online Softmax
  为什么要重缩放旧的和"; "两个融合算子：RMSNorm 与 online softmax"
  (daleiyang.github.io), section "二、递推式怎么来的".
* The merge of two partial pairs,
  (m1, d1) (+) (m2, d2) = (m, d1 * exp(m1 - m) + d2 * exp(m2 - m)), m = max(m1, m2),
  associative and commutative with identity (-inf, 0).
  Same daleiyang page, section "三、结合律：为什么能做树形归约"; notes.kuangjux.top
  section "从逐元素更新到合并两个 tile".

-inf entries (masked keys) contribute exp(-inf) = 0.  When both sides of a
step have m = -inf the formula would evaluate -inf - (-inf) = NaN; the pair
is then the identity (-inf, 0) (the summary of an empty or fully masked
set), which is what the guard returns.
"""
import math

NEG_INF = float("-inf")
IDENTITY = (NEG_INF, 0.0)


def merge(a, b):
    """(m1, d1) (+) (m2, d2) in fp64."""
    m = max(a[0], b[0])
    if m == NEG_INF:
        return IDENTITY
    return (m, a[1] * math.exp(a[0] - m) + b[1] * math.exp(b[0] - m))


def online_stats(xs):
    """Run the element recurrence over xs from the identity; returns (m, d)."""
    m, d = IDENTITY
    for x in xs:
        m_new = max(m, x)
        if m_new == NEG_INF:
            continue  # a masked element before any finite one: still the identity
        d = d * math.exp(m - m_new) + math.exp(x - m_new)
        m = m_new
    return m, d


def element_summary(x):
    """Summary pair of the one-element set {x}."""
    return IDENTITY if x == NEG_INF else (x, 1.0)


def normalise(xs, m, d):
    """y_j = exp(x_j - m) / d (NaN when the row is fully masked)."""
    out = []
    for x in xs:
        if m == NEG_INF:
            out.append(float("nan"))
        else:
            out.append(math.exp(x - m) / d)
    return out


def online_softmax(xs):
    m, d = online_stats(xs)
    return normalise(xs, m, d)


def all_bracketings(pairs):
    """Every way to fold a sequence of pairs with (+), keeping their order.

    Yields one (m, d) result per binary tree over the sequence (a Catalan
    number of them), for brute-force associativity checks on tiny inputs.
    """
    n = len(pairs)
    if n == 1:
        yield pairs[0]
        return
    for split in range(1, n):
        for left in all_bracketings(pairs[:split]):
            for right in all_bracketings(pairs[split:]):
                yield merge(left, right)
