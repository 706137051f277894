"""Input generators: the per-learner draw that the free-running trajectory test
uses is the one build_learners subtracts (CPU)."""
import torch

import workloads


def test_learner_delta_is_the_draw_build_learners_uses():
    for key, ids in (("c3", [1, 2, 3]), ("c5k1", [0, 2995])):
        cfg = workloads.config(key)
        sig = workloads.tensor_sigmas(cfg, len(cfg.tensors))
        theta, _, offs = workloads.build_global(cfg, ids, "cpu", step=2)
        tl, loffs, _ = workloads.build_learners(cfg, ids, theta, offs, "cpu", step=2, sigmas=[sig[t] for t in ids])
        for j, t in enumerate(ids):
            n = cfg.tensors[t].numel
            for i in range(cfg.n_learners):
                d = workloads.learner_delta(cfg, t, i, 2, sig[t], "cpu")
                assert torch.equal(tl[i, loffs[j]:loffs[j] + n], theta[offs[j]:offs[j] + n] - d), (key, t, i)
