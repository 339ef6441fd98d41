"""Calibrate the draft-noise sigma of the synthetic workloads to a target acceptance rate.

Test/bench infrastructure: calls only the oracle.  For a target row z (the workload's
recipe) and a draft row z + sigma * N(0, 1), alpha = sum_v min(p(v), q(v)) with
p = softmax(z / T), q = softmax(zd / T) (the token-level acceptance rate of the
closed form on the lesson page "Decodificação Especulativa e EAGLE", "Aceleração
Esperada").  Bisects sigma so that the mean alpha over `rows` rows hits the target.

    python -m oracle.calibrate_sigma      # prints the table used by the workloads
"""
import numpy as np

from oracle import spec_verify_oracle as O


def target_rows(rng, rows, V, peaks):
    z = rng.normal(0.0, 3.0, (rows, V))
    for r in range(rows):
        if peaks:
            z[r, rng.choice(V, peaks, replace=False)] += 8.0
    return z


def mean_alpha(z, sigma, T, seed):
    rng = np.random.default_rng(seed)
    a = []
    for row in z:
        zd = row + sigma * rng.normal(0.0, 1.0, row.shape)
        a.append(O.acceptance_rate(O.softmax_t(row, T), O.softmax_t(zd, T)))
    return float(np.mean(a))


def calibrate(target, V, T, peaks, rows=24, seed=0):
    z = target_rows(np.random.default_rng(seed), rows, V, peaks)
    lo, hi = 1e-3, 10.0  # alpha decreases in sigma
    for _ in range(40):
        mid = (lo * hi) ** 0.5
        if mean_alpha(z, mid, T, seed + 1) > target:
            lo = mid
        else:
            hi = mid
    s = (lo * hi) ** 0.5
    return s, mean_alpha(z, s, T, seed + 2)


def main():
    cases = [
        ("peaked rows V=128256 T=0.7", 0.8, 128256, 0.7, 16),
        ("plain rows V=262144 T=1", 0.5, 262144, 1.0, 0),
        ("plain rows V=262144 T=1", 0.8, 262144, 1.0, 0),
        ("plain rows V=262144 T=1", 0.95, 262144, 1.0, 0),
    ]
    for name, target, V, T, peaks in cases:
        s, check = calibrate(target, V, T, peaks)
        print(f"{name:32s} alpha={target:.2f}  sigma={s:.4f}  (held-out alpha {check:.4f})")


if __name__ == "__main__":
    main()
